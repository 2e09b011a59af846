"""Decode-step benchmark on one MI355X.

One step = the whole decode hot path for one batch: the slot of each
sequence's newest token, the write of its K/V into the pool, and paged
attention over every context token.  By default the step is one call of
pa_append_decode (pa_append_decode_fp8 for E4M3 pools), which does all three
in one launch (plus the log-sum-exp merge launch when partitions split a
context); ``--step three`` times the same step as pa_compute_slots +
pa_cache_write(_fp8) + pa_decode(_fp8).

Prints ONE JSON line.  By default the line is the largest workload that fits
one GPU: 8 sequences of 32,768 tokens (LLaMA-7B-shaped heads, fp16, blocks of
64) whose first 2048 tokens are one shared prefix, in 512-token partitions.
Every other workload (the tiny fp32 case, the LLaMA-7B layer, the LLaMA-13B
layer at block sizes 16/32/64, the 70B-style grouped-query share, and the
LLaMA-7B and grouped-query shapes over E4M3 pools) is timed in the same run
and reported under ``sub_records``, each with its own roofline.

``value`` is context tokens per second (sum of context_lens over a step / step
time) with every input already in HBM.  ``roofline`` rates the decode launch:
algorithmic bytes (K and V of every context token, q, out, and the used
block-table entries) over its mean duration, measured with HIP events on the
stream the kernels run on (around runs of five timed steps, or every fifth
decode call of the three-call step), against the MI355X HBM peak of 8 TB/s.
``cpu_baseline`` times the float64 oracle on a bounded sample of the same
workload on this host's cores, before the GPU is touched.

Pools are rotated between steps (several resident copies, each larger than
the 256 MB last-level cache together with its neighbours), so a step never
finds the previous step's K/V in cache.

    python bench.py [--steps K] [--warmup W] [--config N] [--sub-configs LIST]
    python bench.py --op {prefill,cache_write,copy_blocks,block_manager}
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn decode: context tokens/s + achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
EVENT_EVERY = 5           # timed steps per HIP-event-timed decode call
MALL_BYTES = 256 << 20
ELEM = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}

# HBM traffic of one pa_decode call, from two rocprofv3 --pmc runs of this
# script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, summed over the
# kernels of the call), each scaled by what the same counter reads for a
# plain 1 GiB device copy in the same run (FETCH_SIZE reads 524,300-524,320
# KiB for the copy's 1,048,576 KiB of reads: factor ~1.9999; WRITE_SIZE
# reads the copy's writes exactly: factor 1.0).  An entry holds only for the kernel
# sources it was taken on (``sources`` = kernel_source_digest()); any change
# to them reports traffic as null until the counters are taken again.
COUNTERS = {
    "longctx_prefix_f16/B64/P512/append": {
        "sources": "321b93fa98b1f2d6220ac623acdd1e1e93ddd87176427f2a6f5a1e190b251427",
        "fetch_kib": 1996293.396 + 4253.500, "fetch_scale": 1048576 / 524318.688,
        "write_kib": 9344.000 + 64.000, "write_scale": 1048576 / 1048576.000,
        "profile": "profiles/decode_counters_all_workloads.md"},
    "tiny_f32/B16/P256/append": {
        "sources": "321b93fa98b1f2d6220ac623acdd1e1e93ddd87176427f2a6f5a1e190b251427",
        "fetch_kib": 902.833, "fetch_scale": 1048576 / 524308.125,
        "write_kib": 24.000, "write_scale": 1048576 / 1048576.000,
        "profile": "profiles/decode_counters_all_workloads.md"},
    "llama7b_f16/B16/P4096/append": {
        "sources": "321b93fa98b1f2d6220ac623acdd1e1e93ddd87176427f2a6f5a1e190b251427",
        "fetch_kib": 328581.667, "fetch_scale": 1048576 / 524308.062,
        "write_kib": 768.000, "write_scale": 1048576 / 1048576.000,
        "profile": "profiles/decode_counters_all_workloads.md"},
    "llama13b_bf16/B16/P4096/append": {
        "sources": "321b93fa98b1f2d6220ac623acdd1e1e93ddd87176427f2a6f5a1e190b251427",
        "fetch_kib": 1311891.875, "fetch_scale": 1048576 / 524313.750,
        "write_kib": 1920.000, "write_scale": 1048576 / 1048576.000,
        "profile": "profiles/decode_counters_all_workloads.md"},
    "llama13b_bf16/B32/P4096/append": {
        "sources": "321b93fa98b1f2d6220ac623acdd1e1e93ddd87176427f2a6f5a1e190b251427",
        "fetch_kib": 1311827.156, "fetch_scale": 1048576 / 524307.438,
        "write_kib": 1920.000, "write_scale": 1048576 / 1048576.000,
        "profile": "profiles/decode_counters_all_workloads.md"},
    "llama13b_bf16/B64/P4096/append": {
        "sources": "321b93fa98b1f2d6220ac623acdd1e1e93ddd87176427f2a6f5a1e190b251427",
        "fetch_kib": 1311795.740, "fetch_scale": 1048576 / 524307.375,
        "write_kib": 1920.000, "write_scale": 1048576 / 1048576.000,
        "profile": "profiles/decode_counters_all_workloads.md"},
    "gqa70b_bf16/B16/P2048/append": {
        "sources": "321b93fa98b1f2d6220ac623acdd1e1e93ddd87176427f2a6f5a1e190b251427",
        "fetch_kib": 103365.875 + 606.333, "fetch_scale": 1048576 / 524314.875,
        "write_kib": 1104.161 + 256.000, "write_scale": 1048576 / 1048576.000,
        "profile": "profiles/decode_counters_all_workloads.md"},
    "llama7b_fp8kv/B16/P4096/append": {
        "sources": "321b93fa98b1f2d6220ac623acdd1e1e93ddd87176427f2a6f5a1e190b251427",
        "fetch_kib": 154701.083, "fetch_scale": 1048576 / 524307.938,
        "write_kib": 512.000, "write_scale": 1048576 / 1048576.000,
        "profile": "profiles/decode_counters_all_workloads.md"},
    "gqa70b_fp8kv/B16/P1024/append": {
        "sources": "321b93fa98b1f2d6220ac623acdd1e1e93ddd87176427f2a6f5a1e190b251427",
        "fetch_kib": 49056.146 + 975.333, "fetch_scale": 1048576 / 524307.375,
        "write_kib": 1824.188 + 256.000, "write_scale": 1048576 / 1048576.000,
        "profile": "profiles/decode_counters_all_workloads.md"},
}


def algorithmic_bytes(context_lens, num_heads, num_kv_heads, head_dim, block_size, dtype,
                      kv_dtype=None, new_row_write=False) -> dict:
    """Bytes a decode launch must move at minimum: K and V rows of every
    context token (per kv head), q and out (per query head) and the 4-byte
    table entries in use.  Per token per kv head K+V is 2*D*e bytes, the
    per-layer form of the KV size formula (2 x tokens x heads x head_dim x
    element bytes).  ``new_row_write``: the launch also stores the newest
    token's K and V rows into the pool (pa_append_decode), 2*D*e bytes per
    sequence and kv head (that token's rows are read from the input instead
    of the pool, the same bytes)."""
    e = ELEM[dtype]
    ekv = ELEM[kv_dtype or dtype]
    ctx = [int(c) for c in context_lens]
    kv = sum(ctx) * num_kv_heads * head_dim * ekv * 2
    qo = 2 * len(ctx) * num_heads * head_dim * e
    table = sum(-(-c // block_size) for c in ctx) * 4
    write = sum(1 for c in ctx if c > 0) * num_kv_heads * head_dim * ekv * 2 if new_row_write else 0
    return {"kv": kv, "q_out": qo, "table": table, "kv_write": write,
            "total": kv + qo + table + write}


# Sources the decode launches are built from (kernels, the headers they
# include, the dispatch) and the build flags: the stored counters hold while
# these are unchanged.
DECODE_SOURCES = ("decode_mha.hip", "decode_gqa.hip", "pa_device.h", "pa_mfma.h",
                  "pa_internal.h", "pa_abi.cpp")


def kernel_source_digest() -> str:
    """sha256 over the decode kernels' sources and the build flags of libpa.so,
    with comments and whitespace taken out (a comment edit does not change
    what was measured)."""
    import hashlib
    import re
    pkg = os.path.join(ROOT, "paged_kv_cache_368_amd")
    csrc = os.path.join(pkg, "csrc")
    h = hashlib.sha256()
    sources = [os.path.join(csrc, f) for f in DECODE_SOURCES]
    for path in sources + [os.path.join(pkg, "build.py")]:
        with open(path) as f:
            text = f.read()
        if path.endswith(".py"):
            text = re.sub(r"#[^\n]*", "", text)
        else:
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
        h.update(os.path.basename(path).encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(workload: str, block_size: int, partition_size: int, fused: bool = False):
    """HBM bytes per decode call (pa_append_decode when ``fused``, else
    pa_decode) from the stored counters, or None when none were taken for
    this workload on the current kernel sources."""
    c = COUNTERS.get(f"{workload}/B{block_size}/P{partition_size}" + ("/append" if fused else ""))
    if c is None or c["sources"] != kernel_source_digest():
        return None
    return (c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024



# ---------------------------------------------------------------------------
# The oracle on the host's cores.  Every CPU baseline runs the oracle as it
# stands, one work item per call, in a pool of forked worker processes (one
# BLAS thread each), before anything in this process has initialised the GPU:
# forking a process that holds GPU state is not safe.
# ---------------------------------------------------------------------------

_ORACLE_STATE = {}          # what the forked workers read (set before the fork)
MAX_HOST_WORKERS = 16       # a one-GPU machine's share of a multi-GPU host's cores


def host_workers() -> tuple[int, int]:
    """(workers to use, cores this process may run on): the affinity set,
    capped at OMP_NUM_THREADS when that is set and at MAX_HOST_WORKERS."""
    aff = len(os.sched_getaffinity(0))
    n = min(aff, MAX_HOST_WORKERS)
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n), aff


def _cpu_name() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _worker_init() -> None:
    """One BLAS thread per worker; arrays the oracle writes (named in
    ``_ORACLE_STATE["private"]``) become private, touched copies before the
    timed region, so no copy-on-write fault lands inside it."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:                                    # pragma: no cover
        pass
    for k in _ORACLE_STATE.get("private", ()):
        _ORACLE_STATE[k] = _ORACLE_STATE[k].copy()


def _run_item(item):
    """One oracle work item in a worker: returns what it counts toward the
    rate (tokens, bytes, ...)."""
    return _ORACLE_STATE["fn"](item)


def parallel_oracle(fn, items, budget_s: float) -> dict:
    """Run ``fn(item)`` over ``items`` (cycled) on the host's cores until
    ``budget_s`` of wall time is spent; ``fn`` returns the item's count.
    Returns the items done, the summed count, the wall seconds, the workers
    and the affinity core count."""
    import itertools
    import multiprocessing as mp

    workers, aff = host_workers()
    _ORACLE_STATE["fn"] = fn
    it = itertools.cycle(items)
    done = acc = 0
    batch = workers * 2
    try:
        with mp.get_context("fork").Pool(workers, initializer=_worker_init) as pool:
            pool.map(_run_item, [items[0]] * workers, chunksize=1)     # start every worker
            t0 = time.perf_counter()
            while True:
                b0 = time.perf_counter()
                chunk = [next(it) for _ in range(batch)]
                acc += sum(pool.map(_run_item, chunk, chunksize=1))
                done += len(chunk)
                now = time.perf_counter()
                if now - t0 > budget_s:
                    break
                if now - b0 < 0.25:
                    batch *= 2
            el = time.perf_counter() - t0
    finally:
        _ORACLE_STATE.clear()
    return {"items": done, "count": acc, "seconds": el, "workers": workers, "affinity": aff}


def _oracle_record(value, unit, run, what) -> dict:
    return {"value": value, "unit": unit, "cores": run["workers"], "kind": "oracle",
            "sample": f"{what}; {run['workers']} worker processes (1 BLAS thread each; "
                      f"{run['affinity']} cores in this process's affinity set) for "
                      f"{run['seconds']:.1f} s on {_cpu_name()}"}


def _decode_pair(item):
    import oracle.paged as P
    wl = _ORACLE_STATE["wl"]
    s, h = item
    if wl.pool_dtype == "fp8":
        P.paged_decode_fp8(wl.q, wl.key_cache, wl.value_cache, wl.block_tables,
                           wl.context_lens, wl.block_size, wl.scale, wl.dtype,
                           wl.k_scale, wl.v_scale, wl.num_kv_heads, pairs=[(s, h)])
    else:
        P.paged_decode(wl.q, wl.key_cache, wl.value_cache, wl.block_tables,
                       wl.context_lens, wl.block_size, wl.scale, wl.dtype,
                       wl.num_kv_heads, pairs=[(s, h)])
    return int(wl.context_lens[s])


def cpu_baseline(wl, budget_s: float = 12.0) -> dict:
    """The float64 oracle as it stands on the workload's (sequence, head)
    pairs in order, cycled until ``budget_s`` is spent, on the host's cores;
    reported as context tokens/s (one context token covers all H heads)."""
    _ORACLE_STATE["wl"] = wl
    pairs = [(s, h) for s in range(wl.num_seqs) for h in range(wl.num_heads)]
    try:
        run = parallel_oracle(_decode_pair, pairs, budget_s)
    finally:
        _ORACLE_STATE.pop("wl", None)
    rate = run["count"] / wl.num_heads / run["seconds"]
    what = (f"{run['items']} (sequence, head) pairs of {wl.name} in order over its "
            f"{len(pairs)} ({run['items'] / len(pairs):.2f} passes), {run['count']} head-tokens, "
            f"float64 numpy")
    return _oracle_record(rate, "context tokens/s", run, what)


# ---------------------------------------------------------------------------
# Decode (the headline): one step = pa_append_decode(_fp8), or the three-call
# step, over one batch of the workload.
# ---------------------------------------------------------------------------

# The largest workload that fits one GPU, timed by default: 8 sequences of
# 32,768 tokens sharing a 2048-token prefix, split into 512-token partitions.
HEADLINE_CONFIG = 4
# Timed in the same run as sub-records: workload[:block size].
SUB_CONFIGS = "0,1,2:16,2:32,2:64,3,5,6"


def parse_sub_configs(spec: str) -> list:
    out = []
    for part in (p.strip() for p in spec.split(",") if p.strip()):
        idx, _, b = part.partition(":")
        out.append((int(idx), int(b) if b else None))
    return out


class ReadProbe:
    """pa_read_probe over one 2 GiB device buffer: the achievable read rate
    in index order, as random 4 KB tiles, and as a call's own tiles over as
    many bytes as its K and V."""

    def __init__(self, torch, pa):
        self.torch, self.pa = torch, pa
        self.big = torch.ones(1 << 29, dtype=torch.int32, device="cuda")
        self.sink = torch.empty(pa.PA_READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")

    def best_gbps(self, buf, tile, order, reps=5) -> float:
        torch, pa = self.torch, self.pa
        stream = torch.cuda.current_stream()
        pa.pa_read_probe(buf, tile, order, self.sink)
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pa.pa_read_probe(buf, tile, order, self.sink)
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 1e3)
        return buf.numel() * 4 / best / 1e9

    def same_bytes(self, kv_bytes: int, tile: int, calls: int = 12) -> float:
        """Mean rate of ``calls`` cold reads of ``kv_bytes`` as random tiles.

        Each call reads the next slice of the 2 GiB buffer, so that (like the
        timed decode steps, which rotate pool copies) no call finds its bytes
        in the last-level cache: re-reading one 100 MB slice measured ~25%
        faster than reading it cold."""
        torch, pa = self.torch, self.pa
        n = max(1, min(kv_bytes // tile, self.big.numel() * 4 // tile))
        perm = torch.randperm(n, device="cuda",
                              generator=torch.Generator(device="cuda").manual_seed(1)).int()
        words = n * tile // 4
        slices = self.big.numel() // words
        stream = torch.cuda.current_stream()
        pa.pa_read_probe(self.big[:words], tile, perm, self.sink)
        total = 0.0
        for i in range(1, calls + 1):
            k = i % slices
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pa.pa_read_probe(self.big[k * words:(k + 1) * words], tile, perm, self.sink)
            e1.record(stream)
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1) / 1e3
        return n * tile * calls / total / 1e9

    def full(self, kv_bytes: int, tile: int) -> dict:
        torch = self.torch
        perm = torch.randperm(self.big.numel() * 4 // 4096, device="cuda",
                              generator=torch.Generator(device="cuda").manual_seed(0)).int()
        return {"how": "pa_read_probe, best of 5 HIP-event-timed calls: 2 GiB in index "
                       "order, 2 GiB as random 4 KB tiles; the call's K+V bytes as its own "
                       "tiles in random order, mean of 12 calls that each read another slice "
                       "of the 2 GiB (cold in the last-level cache, as the decode steps are)",
                "same_bytes_tile_bytes": tile,
                "contiguous_gbps": self.best_gbps(self.big, 4096, None),
                "random_4k_tiles_gbps": self.best_gbps(self.big, 4096, perm),
                "random_tiles_same_bytes_gbps": self.same_bytes(kv_bytes, tile)}


def time_decode(wl, args, torch, pa) -> dict:
    """Time ``args.steps`` decode steps of ``wl`` (after ``args.warmup``
    untimed ones) with its inputs resident in HBM; returns its record."""
    from workloads import to_device

    S, H, Hkv, D, B = wl.num_seqs, wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    dt = wl.dtype
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]
    maxctx = wl.max_context_len
    fp8 = wl.pool_dtype == "fp8"
    size_dt = pa.PA_FP8_E4M3 if fp8 else pa.DTYPE_CODES[tdt]
    lib = pa.load_library()
    P_used = lib.pa_decode_partition_size(S, H, Hkv, D, B, maxctx, wl.partition_size, size_dt)
    ws_bytes = lib.pa_decode_workspace_size(S, H, Hkv, D, B, maxctx, wl.partition_size, size_dt)
    fused = args.step == "fused"
    nbytes = algorithmic_bytes(wl.context_lens, H, Hkv, D, B, dt, wl.pool_dtype,
                               new_row_write=fused)
    sum_ctx = int(wl.context_lens.sum())

    base = to_device(wl)
    pool_bytes = base.key_cache.numel() * base.key_cache.element_size() * 2
    # Rotate pool copies so that no step finds the previous one's K/V in the
    # 256 MB last-level cache.
    copies = max(2, math.ceil(2 * MALL_BYTES / pool_bytes) + 1)
    pools = [(base.key_cache, base.value_cache)] + [
        (base.key_cache.clone(), base.value_cache.clone()) for _ in range(copies - 1)]
    slots = torch.empty(S, dtype=torch.int64, device="cuda")
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: S={S} H={H}/{Hkv} D={D} B={B} {dt}"
          f"{' K/V fp8' if fp8 else ''} sum(ctx)={sum_ctx} P={P_used} pool copies={copies} "
          f"({pool_bytes / 2**20:.0f} MiB each)", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        kc, vc = pools[i % copies]
        if fused:
            if fp8:
                pa.pa_append_decode_fp8(base.out, base.q, base.new_key, base.new_value, kc, vc,
                                        base.block_tables, base.context_lens, maxctx,
                                        wl.k_scale, wl.v_scale, wl.scale, wl.partition_size,
                                        workspace)
            else:
                pa.pa_append_decode(base.out, base.q, base.new_key, base.new_value, kc, vc,
                                    base.block_tables, base.context_lens, maxctx, wl.scale,
                                    wl.partition_size, workspace)
            return
        pa.pa_compute_slots(slots, base.block_tables, B, wl.num_blocks,
                            context_lens=base.context_lens)
        if fp8:
            pa.pa_cache_write_fp8(base.new_key, base.new_value, kc, vc, slots, wl.k_scale,
                                  wl.v_scale)
        else:
            pa.pa_cache_write(base.new_key, base.new_value, kc, vc, slots)
        if ev is not None:
            ev[0].record(stream)
        if fp8:
            pa.pa_decode_fp8(base.out, base.q, kc, vc, base.block_tables, base.context_lens,
                             maxctx, wl.k_scale, wl.v_scale, wl.scale, wl.partition_size,
                             workspace)
        else:
            pa.pa_decode(base.out, base.q, kc, vc, base.block_tables, base.context_lens, maxctx,
                         wl.scale, wl.partition_size, workspace)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Launch durations from HIP events on the kernels' stream.  One-launch
    # steps: an event pair brackets each run of EVENT_EVERY consecutive steps
    # (launch duration = elapsed / run length), so the events' own cost (~8 us
    # per pair on a ~105 us LLaMA-7B step) is paid once per run.  Three-call
    # steps: the pair brackets the decode call of every EVENT_EVERY-th step.
    # Fewer than 2 * EVENT_EVERY timed steps: every step is measured alone.
    every = EVENT_EVERY if args.steps >= 2 * EVENT_EVERY else 1
    samples = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if fused:
        for g0 in range(0, args.steps, every):
            g1 = min(g0 + every, args.steps)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(g0, g1):
                step(args.warmup + i)
            e1.record(stream)
            samples.append((e0, e1, g1 - g0))
    else:
        for i in range(args.steps):
            if i % every == 0:
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                samples.append((ev[0], ev[1], 1))
                step(args.warmup + i, ev)
            else:
                step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = sorted(e0.elapsed_time(e1) / n for e0, e1, n in samples)
    dec_mean_s = sum(dec_ms) / len(dec_ms) / 1e3
    dec_med_s = dec_ms[len(dec_ms) // 2] / 1e3
    print(f"[bench] {wl.name}: {args.steps} steps in {wall * 1e3:.2f} ms; decode mean "
          f"{dec_mean_s * 1e6:.1f} us median {dec_med_s * 1e6:.1f} us p10 "
          f"{dec_ms[len(dec_ms) // 10] * 1e3:.1f} us p90 "
          f"{dec_ms[(9 * len(dec_ms)) // 10] * 1e3:.1f} us", file=sys.stderr, flush=True)
    del pools, base, workspace, slots
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    achieved = nbytes["total"] / dec_mean_s / 1e9
    # which kernels the library dispatches to (for the record's label only)
    gqa = wl.pool_dtype in ("f16", "bf16", "fp8") and H // Hkv >= 2
    kernels = ("decode_gqa_kernel" if gqa else "decode_mha_kernel") + (
        " + merge_kernel" if P_used < maxctx else "")
    return {
        "workload": wl.name,
        "value": sum_ctx * args.steps / wall,
        "unit": "context tokens/s",
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "dtype": dt if not fp8 else f"{dt} (K/V fp8 e4m3)",
        "config": {"workload": wl.name, "num_seqs": S, "num_heads": H, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": B, "sum_context_tokens": sum_ctx,
                   "max_context_len": maxctx, "partition_size": P_used, "seed": wl.seed,
                   "pool_copies_rotated": copies,
                   "step": ("pa_append_decode(_fp8): slot, K/V write and attention in one "
                            "launch" if fused else "pa_compute_slots + pa_cache_write(_fp8) + "
                            "pa_decode(_fp8)")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(wl.name, B, P_used, fused),
                     "kernel": ("pa_append_decode" if fused else "pa_decode") +
                               ("_fp8" if fp8 else "") + f" ({kernels})",
                     "bytes_per_launch": nbytes["total"], "mean_launch_us": dec_mean_s * 1e6,
                     "median_launch_us": dec_med_s * 1e6, "event_samples": len(dec_ms),
                     "launches_per_sample": every if fused else 1,
                     "p10_launch_us": dec_ms[len(dec_ms) // 10] * 1e3,
                     "p90_launch_us": dec_ms[(9 * len(dec_ms)) // 10] * 1e3},
        "decode_context_tokens_per_s": sum_ctx / dec_mean_s,
        "_kv_bytes": nbytes["kv"],
        "_tile_bytes": max(1024, B * D * ELEM[wl.pool_dtype or dt]),
    }


def bench_decode(args) -> dict:
    """The headline line (one workload, by default the long-context one) and
    the sub-records of the other workloads, timed in one run."""
    from workloads import make_workload

    head_idx = HEADLINE_CONFIG if args.config is None else args.config
    subs = []
    if args.sub_configs is not None:
        subs = parse_sub_configs(args.sub_configs)
    elif args.config is None:
        subs = parse_sub_configs(SUB_CONFIGS)
    print(f"[bench] building workload {head_idx}", file=sys.stderr, flush=True)
    wl = make_workload(head_idx, seed=args.seed, block_size=args.block_size)
    if args.partition_size is not None:
        wl.partition_size = args.partition_size
    cpu = None
    if not args.no_cpu_baseline:
        # before this process touches the GPU (the oracle runs in forked workers)
        print(f"[bench] timing the float64 oracle on the host ({host_workers()[0]} workers)",
              file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl)

    import torch

    import paged_kv_cache_368_amd as pa
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pa.load_library()
    dev_name = torch.cuda.get_device_name(0)
    print(f"[bench] device {dev_name}", file=sys.stderr, flush=True)
    head = time_decode(wl, args, torch, pa)
    del wl
    probe = None
    ceiling = None
    if not args.no_ceiling:
        probe = ReadProbe(torch, pa)
        ceiling = probe.full(head["_kv_bytes"], head["_tile_bytes"])

    records = []
    for idx, b in subs:
        print(f"[bench] building workload {idx}" + (f" (B={b})" if b else ""), file=sys.stderr,
              flush=True)
        swl = make_workload(idx, block_size=b)
        rec = time_decode(swl, args, torch, pa)
        del swl
        if probe is not None:
            rec["random_tiles_same_bytes_gbps"] = probe.same_bytes(rec["_kv_bytes"],
                                                                   rec["_tile_bytes"])
            rec["frac_of_same_bytes_tile_ceiling"] = (rec["roofline"]["achieved"] /
                                                      rec["random_tiles_same_bytes_gbps"])
        for k in ("_kv_bytes", "_tile_bytes"):
            rec.pop(k)
        records.append(rec)
    if probe is not None:
        del probe
        torch.cuda.synchronize()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    achieved = head["roofline"]["achieved"]
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "context tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) K/V/q, random block tables; no dataset)",
        "config": head["config"],
        "roofline": head["roofline"],
        "read_ceiling": ceiling,
        "frac_of_tile_ceiling": (achieved / ceiling["random_4k_tiles_gbps"]) if ceiling else None,
        "frac_of_same_bytes_tile_ceiling":
            (achieved / ceiling["random_tiles_same_bytes_gbps"]) if ceiling else None,
        "decode_context_tokens_per_s": head["decode_context_tokens_per_s"],
        "device": dev_name,
        "cpu_baseline": cpu,
        "sub_records": records,
    }
    return result


# ---------------------------------------------------------------------------
# Other ops, each on its own line (--op ...)
# ---------------------------------------------------------------------------

def _copy_item(pair):
    import oracle.paged as P
    kc, vc = _ORACLE_STATE["kc"], _ORACLE_STATE["vc"]
    P.copy_blocks(kc, kc, [pair])
    P.copy_blocks(vc, vc, [pair])
    return 2 * 2 * kc[0].nbytes                  # read + write, K and V


def _copy_cpu_baseline(Hkv, B, D, npairs) -> dict:
    """The oracle's block copy on host pools of the same block shape: copy
    on write of a random pairing's pairs, bytes read + written."""
    import numpy as np

    NB = 2 * npairs
    rng = np.random.default_rng(11)
    _ORACLE_STATE["kc"] = rng.integers(0, 65535, (NB, Hkv, B, D), dtype=np.uint16)
    _ORACLE_STATE["vc"] = rng.integers(0, 65535, (NB, Hkv, B, D), dtype=np.uint16)
    _ORACLE_STATE["private"] = ("kc", "vc")
    perm = rng.permutation(NB)
    pairs = list(zip(perm[:npairs].tolist(), perm[npairs:].tolist()))
    try:
        run = parallel_oracle(_copy_item, pairs, 10.0)
    finally:
        for k in ("kc", "vc", "private"):
            _ORACLE_STATE.pop(k, None)
    return _oracle_record(run["count"] / run["seconds"] / 1e9, "GB/s (read+write)", run,
                          f"{run['items']} block pairs of {npairs} (K and V), numpy")


def bench_copy_blocks(args) -> dict:
    """Whole-block copies (pa_copy_blocks) on LLaMA-13B-shaped bf16 pools
    (40 kv heads x 16 tokens x 128 dims = 160 KB per block and pool):
    copy on write of --pairs random blocks inside the device pools, and a
    swap of the same number of blocks out to pinned host memory and back.
    Bytes = read + write of both pools."""
    Hkv, B, D, npairs = 40, 16, 128, args.pairs
    # the host sample: 512 pairs over 1024 blocks per pool (each worker holds
    # its own copy of the pools it writes)
    cpu = None if args.no_cpu_baseline else _copy_cpu_baseline(Hkv, B, D, min(npairs, 512))

    import torch

    import paged_kv_cache_368_amd as pa
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    NB = max(4 * npairs, 8192)
    block_bytes = Hkv * B * D * 2
    g = torch.Generator().manual_seed(11)
    kc = torch.randn((NB, Hkv, B, D), generator=g).to(torch.bfloat16).cuda()
    vc = torch.randn((NB, Hkv, B, D), generator=g).to(torch.bfloat16).cuda()
    perm = torch.randperm(NB, generator=g)
    pairs = torch.stack([perm[:npairs], perm[npairs:2 * npairs]], 1).to(torch.int32).cuda()
    host_k = torch.empty((npairs, Hkv, B, D), dtype=torch.bfloat16, pin_memory=True)
    host_v = torch.empty_like(host_k, pin_memory=True)
    out_pairs = torch.stack([perm[:npairs], torch.arange(npairs)], 1).to(torch.int32).cuda()
    in_pairs = torch.stack([torch.arange(npairs), perm[2 * npairs:3 * npairs]], 1).to(torch.int32).cuda()
    torch.cuda.synchronize()

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in ev)
        return sum(ts) / len(ts)

    moved = 2 * 2 * npairs * block_bytes          # read + write, K and V
    t_cow = timed(lambda: pa.pa_copy_blocks(kc, kc, pairs, vc, vc), args.steps)
    t_out = timed(lambda: pa.pa_copy_blocks(host_k, kc, out_pairs, host_v, vc), max(3, args.steps // 5))
    t_in = timed(lambda: pa.pa_copy_blocks(kc, host_k, in_pairs, vc, host_v), max(3, args.steps // 5))
    one_way = 2 * npairs * block_bytes
    return {
        "metric": "block copy (pa_copy_blocks): copy-on-write GB/s in HBM, swap GB/s over the host link",
        "value": moved / t_cow / 1e9, "unit": "GB/s (read+write)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t_cow * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random bf16 pools, random block pairs)",
        "config": {"workload": "llama13b_bf16_block_copy", "num_kv_heads": Hkv, "block_size": B,
                   "head_dim": D, "pairs": npairs, "block_bytes": block_bytes},
        "roofline": {"bound": "hbm", "achieved": moved / t_cow / 1e9, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": moved / t_cow / 1e9 / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "copy_blocks_kernel (copy on write)", "bytes_per_launch": moved,
                     "mean_launch_us": t_cow * 1e6},
        "swap_out_gbps": one_way / t_out / 1e9, "swap_in_gbps": one_way / t_in / 1e9,
        "swap_out_us": t_out * 1e6, "swap_in_us": t_in * 1e6,
        "cpu_baseline": cpu,
    }


def _cache_write_item(i):
    import oracle.paged as P
    st = _ORACLE_STATE
    P.cache_write(st["kc"], st["vc"], st["key"][i:i + 1], st["val"][i:i + 1],
                  st["slots"][i:i + 1], st["B"])
    return 2 * 2 * st["key"][i].nbytes            # K and V rows read + written


def _cache_write_cpu_baseline(Hkv, B, D) -> dict:
    """The oracle's cache write, one token per call, into host pools of the
    same row shape (1024 blocks) at distinct random slots."""
    import numpy as np

    NB, T = 1024, 16384
    rng = np.random.default_rng(12)
    _ORACLE_STATE.update(
        kc=np.zeros((NB, Hkv, B, D), dtype=np.uint16), vc=np.zeros((NB, Hkv, B, D), dtype=np.uint16),
        key=rng.integers(0, 65535, (T, Hkv, D), dtype=np.uint16),
        val=rng.integers(0, 65535, (T, Hkv, D), dtype=np.uint16),
        slots=rng.permutation(NB * B)[:T].astype(np.int64), B=B, private=("kc", "vc"))
    try:
        run = parallel_oracle(_cache_write_item, list(range(T)), 8.0)
    finally:
        for k in ("kc", "vc", "key", "val", "slots", "B", "private"):
            _ORACLE_STATE.pop(k, None)
    return _oracle_record(run["count"] / run["seconds"] / 1e9, "GB/s (read+write)", run,
                          f"{run['items']} tokens (K and V rows, one per call) of {T}, numpy")


def bench_cache_write(args) -> dict:
    """pa_cache_write on LLaMA-13B-shaped bf16 pools (8192 blocks of 16
    tokens, 40 kv heads of 128): the K/V rows of a prompt batch (8 x 2048
    tokens, the value: GB/s of rows read + slot bytes written) and of one
    decode step (64 tokens, latency), each into distinct random slots."""
    Hkv, B, D, NB = 40, 16, 128, 8192
    cpu = None if args.no_cpu_baseline else _cache_write_cpu_baseline(Hkv, B, D)

    import torch

    import paged_kv_cache_368_amd as pa
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    g = torch.Generator(device="cuda").manual_seed(12)
    kc = torch.empty((NB, Hkv, B, D), dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    vc = torch.empty_like(kc).normal_(generator=g)
    out = {}
    for name, T in (("prompt", 8 * 2048), ("step", 64)):
        key = torch.empty((T, Hkv, D), dtype=torch.bfloat16, device="cuda").normal_(generator=g)
        val = torch.empty_like(key).normal_(generator=g)
        slots = torch.randperm(NB * B, device="cuda", generator=g)[:T].to(torch.int64)
        for _ in range(args.warmup):
            pa.pa_cache_write(key, val, kc, vc, slots)
        torch.cuda.synchronize()
        # One event pair around all the calls: a 64-token write is shorter
        # than what a per-call event pair adds.
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            pa.pa_cache_write(key, val, kc, vc, slots)
        b.record()
        torch.cuda.synchronize()
        mean = a.elapsed_time(b) / args.steps * 1e-3
        moved = 2 * 2 * T * Hkv * D * 2 + T * 8       # rows read + written (K and V), slots read
        out[name] = (T, mean, moved)
    T, t, moved = out["prompt"]
    Ts, ts, moved_s = out["step"]
    # The same kernel and bytes with the prompt's rows going to sorted random
    # slots and to consecutive slots: how much of the time the scattered
    # destinations themselves cost (the rows are written 256 B at a time).
    order = {}
    key = torch.empty((T, Hkv, D), dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    val = torch.empty_like(key).normal_(generator=g)
    rnd = torch.randperm(NB * B, device="cuda", generator=g)[:T].to(torch.int64)
    # Through block tables: each prompt of 2048 tokens fills 128 random
    # blocks in order (token t of a prompt at table[t // B] * B + t % B).
    tables = torch.randperm(NB, device="cuda", generator=g)[:T // B].to(torch.int64)
    tok = torch.arange(T, dtype=torch.int64, device="cuda")
    by_table = tables[tok // B] * B + tok % B
    for name, slots in (("sorted_random_slots", torch.sort(rnd).values),
                        ("block_table_slots", by_table),
                        ("consecutive_slots", tok)):
        for _ in range(args.warmup):
            pa.pa_cache_write(key, val, kc, vc, slots)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            pa.pa_cache_write(key, val, kc, vc, slots)
        b.record()
        torch.cuda.synchronize()
        order[name + "_gbps"] = moved / (a.elapsed_time(b) / args.steps * 1e-3) / 1e9
    return {
        "metric": "KV cache write (pa_cache_write): GB/s of rows read + written into scattered slots",
        "value": moved / t / 1e9, "unit": "GB/s (read+write)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal bf16 rows and pools, distinct random slots)",
        "config": {"workload": "llama13b_bf16_cache_write", "num_kv_heads": Hkv, "block_size": B,
                   "head_dim": D, "num_blocks": NB, "tokens": T},
        "roofline": {"bound": "hbm", "achieved": moved / t / 1e9, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": moved / t / 1e9 / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "cache_write_kernel", "bytes_per_launch": moved,
                     "mean_launch_us": t * 1e6},
        "decode_step_write": {"tokens": Ts, "mean_us": ts * 1e6, "gbps": moved_s / ts / 1e9},
        "slot_order_reference": order,
        "cpu_baseline": cpu,
    }


MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}
PREFILL_WARM_S = 0.3           # seconds of untimed prefill calls before the timed ones


def prefill_flops(context_lens, query_lens, num_heads, head_dim) -> int:
    """Algorithmic flops of causal prefill: each (query row, head) at position
    p does 2*D flops for q.k and 2*D for p*V with each of its p + 1 keys."""
    total = 0
    for n, L in zip(context_lens, query_lens):
        first = int(n) - int(L)
        total += sum(first + j + 1 for j in range(int(L)))
    return 4 * head_dim * num_heads * total


def prefill_workload(prefix: int, fp8: bool):
    """The prefill bench's inputs: 8 LLaMA-7B-shaped prompts of 2048 tokens
    (32 heads of 128, fp16 queries, N(0,1)*0.5 values, blocks of 16, seed 7),
    whose last 2048 - ``prefix`` tokens are the query rows; K/V pools in fp16
    or as E4M3 codes with scale 0.5.  Returns (workload, query_start, q)."""
    import numpy as np

    from workloads import build, normal_array
    S, H, D, B, n = 8, 32, 128, 16, 2048
    L = n - prefix
    wl = build("llama7b_prefill_fp8kv" if fp8 else "llama7b_prefill_f16", "f16", [n] * S, H, H,
               D, B, seed=7, pool="permutation", value_scale=0.5,
               kv_dtype="fp8" if fp8 else None, kv_scale=0.5)
    qs = np.arange(S + 1, dtype=np.int32) * L
    q = normal_array(7, 40, (S * L, H, D), "f16", 0.5)
    return wl, qs, q


def _prefill_item(item):
    import oracle.paged as P
    st = _ORACLE_STATE
    wl, qs, q = st["wl"], st["qs"], st["q"]
    if wl.pool_dtype == "fp8":
        P.paged_prefill_fp8(q, wl.key_cache, wl.value_cache, wl.block_tables,
                            wl.context_lens, qs, wl.block_size, wl.scale, wl.dtype,
                            wl.k_scale, wl.v_scale, wl.num_kv_heads, rows=[item])
    else:
        P.paged_prefill(q, wl.key_cache, wl.value_cache, wl.block_tables, wl.context_lens,
                        qs, wl.block_size, wl.scale, wl.dtype, wl.num_kv_heads, rows=[item])
    return 1


def _prefill_cpu_baseline(wl, qs, q, prefix) -> dict:
    """The float64 oracle's prefill on (row, head) pairs of the same workload
    in a seeded random order (a representative mix of rows), on the host's
    cores; reported as query tokens/s (a query token covers all heads)."""
    import numpy as np

    items = [(i, h) for i in range(int(qs[-1])) for h in range(wl.num_heads)]
    order = np.random.default_rng(0).permutation(len(items))
    items = [items[k] for k in order]
    _ORACLE_STATE.update(wl=wl, qs=qs, q=q)
    try:
        run = parallel_oracle(_prefill_item, items, 12.0)
    finally:
        for k in ("wl", "qs", "q"):
            _ORACLE_STATE.pop(k, None)
    return _oracle_record(run["count"] / wl.num_heads / run["seconds"], "query tokens/s", run,
                          f"{run['items']} of {len(items)} (query row, head) pairs in seeded "
                          f"random order, {prefix}-token cached prefix, float64 numpy")


def bench_prefill(args) -> dict:
    """pa_prefill (pa_prefill_fp8 with --kv fp8) on LLaMA-7B-shaped prompts
    (32 heads of 128, fp16, blocks of 16): 8 sequences of 2048 tokens, either
    whole fresh prompts or the last 512 tokens after a 1536-token cached
    prefix (--prefix)."""
    fp8 = getattr(args, "kv", "f16") == "fp8"
    wl, qs, q_raw = prefill_workload(args.prefix, fp8)
    cpu = None if args.no_cpu_baseline else _prefill_cpu_baseline(wl, qs, q_raw, args.prefix)

    import torch

    import paged_kv_cache_368_amd as pa
    from workloads import to_torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    S, H, D, B = wl.num_seqs, wl.num_heads, wl.head_dim, wl.block_size
    n = wl.max_context_len
    L = n - args.prefix
    q = to_torch(q_raw, "f16", "cuda")
    kc, vc = to_torch(wl.key_cache, wl.pool_dtype, "cuda"), to_torch(wl.value_cache, wl.pool_dtype, "cuda")
    bt = torch.tensor(wl.block_tables, device="cuda")
    cl = torch.tensor(wl.context_lens, device="cuda")
    qst = torch.tensor(qs, device="cuda")
    out = torch.empty_like(q)
    flops = prefill_flops(wl.context_lens, [L] * S, H, D)

    def call():
        if fp8:
            pa.pa_prefill_fp8(out, q, kc, vc, bt, cl, qst, L, n, wl.k_scale, wl.v_scale, wl.scale)
        else:
            pa.pa_prefill(out, q, kc, vc, bt, cl, qst, L, n, wl.scale)
    torch.cuda.synchronize()
    # Warm-up: the requested calls, and then more until PREFILL_WARM_S of them
    # have run: the matrix-core-bound launch runs at the engine clock, which
    # rises over the first ~0.1 s of load (measured on one machine: 405 us per
    # call after 3 warm-up calls, 361 us after 2000; the decode launches,
    # bound by HBM, do not move).
    warm = 0
    t_w = time.perf_counter()
    while warm < args.warmup or time.perf_counter() - t_w < PREFILL_WARM_S:
        for _ in range(10):
            call()
        warm += 10
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e-3
    tflops = flops / mean / 1e12
    entry = "pa_prefill_fp8" if fp8 else "pa_prefill"
    return {
        "metric": f"paged prefill ({entry}): query tokens/s and causal attention TFLOP/s",
        "value": S * L / mean, "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warm, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 (K/V fp8 e4m3)" if fp8 else "f16",
        "data": "synthetic (seeded N(0,1)*0.5 q/K/V, random block tables)",
        "config": {"workload": wl.name, "num_seqs": S, "num_heads": H,
                   "head_dim": D, "block_size": B, "context_len": n, "query_len": L,
                   "cached_prefix": args.prefix, "kv": "fp8 E4M3" if fp8 else "f16"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_PEAK_TFLOPS["f16"],
                     "unit": "TFLOP/s", "frac": tflops / MFMA_PEAK_TFLOPS["f16"], "traffic": None,
                     "kernel": "prefill_kernel", "flops_per_launch": flops,
                     "mean_launch_us": mean * 1e6},
        "cpu_baseline": cpu,
    }


def _bm_replay_lib(bm, events, max_blocks):
    """Send schedule events to the library's block manager (C++ through the
    binding); returns the number of decode-step appends."""
    n = 0
    for ev in events:
        kind = ev[0]
        if kind == "append":
            bm.append_slots(ev[1], ev[2])
        elif kind == "fill":
            bm.fill_tables(ev[1], max_blocks)
            n += len(ev[1])                      # one decode-step append per filled row
        elif kind == "alloc":
            bm.allocate(ev[1], ev[2])
        elif kind == "share":
            bm.share_prefix(ev[1], ev[2], ev[3])
        elif kind == "free":
            bm.free_request(ev[1])
        elif kind == "fork":
            bm.fork(ev[1], ev[2])
    return n


def _bm_replay_oracle(om, ev, max_blocks):
    """One schedule event on the oracle's block manager (plain Python)."""
    import numpy as np
    kind = ev[0]
    if kind == "append":
        for r, p in zip(ev[1].tolist(), ev[2].tolist()):
            om.append_slot(r, p)
    elif kind == "fill":
        out = np.full((len(ev[1]), max_blocks), -1, dtype=np.int32)
        for i, r in enumerate(ev[1].tolist()):
            t = om.table(r)
            out[i, :len(t)] = t
        return len(ev[1])
    elif kind == "alloc":
        om.allocate_for_request(ev[1], ev[2])
    elif kind == "share":
        om.share_prefix_blocks(ev[1], ev[2], ev[3])
    elif kind == "free":
        om.free_request(ev[1])
    elif kind == "fork":
        om.fork(ev[1], ev[2])
    return 0


def bench_block_manager(args) -> dict:
    """The host block manager (include/pa_blocks.h, C++) on a continuous-
    batching decode schedule: 256 live requests, prompts of 512-2048 tokens
    (a quarter start from a shared 1024-token system prompt), 32-256
    generated tokens each, then freed and replaced, occasional beam forks
    (copy on write at the next append); blocks of 16 tokens.  Each decode
    step is one pa_bm_append_slots over the batch and one pa_bm_fill_tables
    (pa_decode's block_tables), through the Python binding as a serving loop
    would call it.  Host only: no GPU is used."""
    import workloads as W
    from paged_kv_cache_368_amd.blocks import BlockManager

    batch, B, NB = 256, 16, 48000
    max_blocks = (2048 + 256) // B + 1
    steps = max(args.steps, 1) * 10
    warm = max(args.warmup, 0) * 10
    setup, per_step = W.block_manager_schedule(5, batch, warm + steps)
    bm = BlockManager(NB, B)
    _bm_replay_lib(bm, setup, max_blocks)
    for ev in per_step[:warm]:
        _bm_replay_lib(bm, ev, max_blocks)
    t0 = time.perf_counter()
    appends = 0
    for ev in per_step[warm:]:
        appends += _bm_replay_lib(bm, ev, max_blocks)
    el = time.perf_counter() - t0
    free, used, nreq = bm.stats()
    bm.close()
    out = {
        "metric": "host block manager: decode-step token appends/s (append_slots + fill_tables "
                  "per step, continuous batching)",
        "value": appends / el, "unit": "appended tokens/s", "n_gpus": 0, "steps": steps,
        "warmup": warm, "ms_per_step": el * 1e3 / steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic seeded request schedule (workloads.block_manager_schedule)",
        "config": {"workload": "block_manager_continuous_batching", "live_requests": batch,
                   "block_size": B, "num_blocks": NB, "prompt_tokens": [512, 2048],
                   "generated_tokens": [32, 256], "shared_system_prompt": 1024,
                   "blocks_in_use_at_end": used, "requests_at_end": nreq},
        "roofline": None,
        "cpu_baseline": None if args.no_cpu_baseline else _bm_cpu_baseline(setup, per_step,
                                                                           NB, B, max_blocks),
    }
    return out


def _bm_cpu_baseline(setup, per_step, NB, B, max_blocks) -> dict:
    """The oracle's block manager (plain Python) on the same schedule from its
    start, until ~10 s are spent.  One manager is one sequence of state
    changes, so this runs on one core (as does the library's manager)."""
    import oracle.blocks as OB
    om = OB.BlockManager(NB, B)
    for ev in setup:
        _bm_replay_oracle(om, ev, max_blocks)
    appends, steps_done = 0, 0
    t0 = time.perf_counter()
    for st in per_step:
        for ev in st:
            appends += _bm_replay_oracle(om, ev, max_blocks)
        steps_done += 1
        if time.perf_counter() - t0 > 10.0:
            break
    el = time.perf_counter() - t0
    return {"value": appends / el, "unit": "appended tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {steps_done} decode steps of the same schedule (after its "
                      f"setup), plain Python, 1 thread (one manager's state changes are "
                      f"sequential) on {_cpu_name()}"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=None,
                    help="time only this workload (0..6) as the line; default: the long-context "
                         f"workload {HEADLINE_CONFIG} as the line, the others as sub_records")
    ap.add_argument("--sub-configs", default=None,
                    help=f"workloads timed as sub_records, e.g. '{SUB_CONFIGS}' (index[:block "
                         "size]); default: those when --config is not given, else none")
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", choices=["decode", "copy_blocks", "prefill", "cache_write",
                                     "block_manager"],
                    default="decode",
                    help="decode (the headline step, default), whole-block copies, prefill, "
                         "the cache write, or the host block manager")
    ap.add_argument("--kv", choices=["f16", "fp8"], default="f16",
                    help="--op prefill: K/V pools in fp16 or as E4M3 codes (pa_prefill_fp8)")
    ap.add_argument("--prefix", type=int, default=0,
                    help="--op prefill: tokens of each 2048-token prompt already cached")
    ap.add_argument("--pairs", type=int, default=2048, help="block pairs for --op copy_blocks")
    ap.add_argument("--step", choices=["fused", "three"], default="fused",
                    help="decode step as one pa_append_decode call (default) or as "
                         "pa_compute_slots + pa_cache_write + pa_decode")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the STREAM-like read ceiling measured after the timed steps")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    run = {"decode": bench_decode, "copy_blocks": bench_copy_blocks, "prefill": bench_prefill,
           "cache_write": bench_cache_write, "block_manager": bench_block_manager}[args.op]
    print(json.dumps(run(args)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
