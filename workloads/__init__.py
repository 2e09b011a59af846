"""Seeded synthetic inputs for paged decode: pools, block tables, queries.

This module is the only code shared by the float64 oracle (``oracle/``) and the
HIP path (``paged_kv_cache_368_amd``).  It draws random numbers and lays them
out; it computes nothing of the attention itself (no scores, no softmax, no
slot resolution for the kernels -- the one place that needs to know which pool
slots hold live tokens, the NaN poisoning of unused slots, walks each table
with its own counter).

Recipe (every array is reproducible from ``seed`` alone):

* Values are standard normals drawn in float32 from numpy ``PCG64`` streams,
  one stream per named array, split into fixed 4 Mi-element chunks whose seeds
  come from ``SeedSequence(seed, spawn_key=(array_id, chunk))`` -- so the result
  does not depend on how many threads draw it.  They are multiplied by the
  workload's value scale (0.5 for the LLaMA-7B shape, else 1) and rounded to
  the storage type with round-to-nearest-even: integer rounding of the
  float32 word to fp16 (the same words as numpy's cast) or to bf16 (stored
  as raw ``uint16``).
* E4M3 pools hold random codes drawn as bit patterns (see ``e4m3_codes``).
* Pools are ``[num_blocks][num_kv_heads][block_size][head_dim]``.  Every slot
  that no sequence's context covers (whole unused blocks and the tail of each
  sequence's last block) is set to NaN, so any kernel that lets a masked slot
  leak into the result produces NaN.
* Block tables are int32 ``[num_seqs][max_blocks_per_seq]`` padded with -1.
* Integer draws are inclusive of both bounds.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

# ids of the named random streams
_STREAM = {"q": 1, "k": 2, "v": 3, "new_k": 4, "new_v": 5, "cw_k": 6, "cw_v": 7}


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    b = x.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (nearest, ties to even); returns uint16
    bits.  The same words as ``x.astype(np.float16)`` for every input (NaN
    becomes 0x7E00), written in integer ufuncs that release the GIL, so the
    chunked draws convert in parallel (numpy's own float16 cast does not)."""
    b = x.view(np.uint32)
    a = b & np.uint32(0x7FFFFFFF)
    # normal binary16 range: rebias the exponent (127 - 15 = 112) and round
    # the 23-bit significand to 10 bits; a carry out of the significand moves
    # into the exponent, and past 65504 the result lands on infinity (0x7C00).
    n = a - np.uint32(112 << 23)
    t = n >> np.uint32(13)
    t &= np.uint32(1)
    n += t
    n += np.uint32(0x0FFF)
    n >>= np.uint32(13)
    np.minimum(n, np.uint32(0x7C00), out=n)
    # below 2^-14: a multiple of 2^-24, exact in float32 after scaling by 2^24
    sub = np.abs(x)
    sub *= np.float32(2.0 ** 24)
    np.rint(sub, out=sub)
    np.copyto(n, sub.astype(np.uint32), where=a < np.uint32(0x38800000))
    np.copyto(n, np.uint32(0x7E00), where=a > np.uint32(0x7F800000))
    h = n.astype(np.uint16)
    h |= (b >> np.uint32(16)).astype(np.uint16) & np.uint16(0x8000)
    return h


def _encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return _f32_to_f16_bits(x32).view(np.float16)
    if dtype == "bf16":
        return _f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def nan_bits(dtype: str):
    """The storage word of a quiet NaN in ``dtype``."""
    if dtype == "fp8":
        return np.uint8(0x7F)
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "f16":
        return np.float16(np.nan)
    return np.uint16(0x7FC0)


def normal_array(seed: int, stream: int, shape, dtype: str, scale: float = 1.0,
                 threads: int | None = None) -> np.ndarray:
    """``scale * N(0, 1)`` draws of ``shape``, stored as ``dtype`` (see module doc)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=STORAGE[dtype])
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, c))))
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[lo:hi] = _encode(x, dtype)

    if threads is None:
        threads = min(8, len(os.sched_getaffinity(0)))
    if nchunks <= 1 or threads <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


# Exponent fields of random E4M3 codes, as a lookup table over 50 equally
# likely draws: magnitudes mostly within a factor of 8 of 1 (fields 4..8 are
# 2^-3 .. 2^1), as a normal sample would be.
_E4M3_EXP_TABLE = np.repeat(np.arange(2, 10, dtype=np.uint8),
                            [1, 2, 4, 8, 14, 14, 6, 1])          # 50 entries


def e4m3_codes(seed: int, stream: int, shape, threads: int | None = None,
               all_codes: bool = False) -> np.ndarray:
    """Random E4M3 storage codes (uint8): random sign and mantissa bits and an
    exponent field drawn from ``_E4M3_EXP_TABLE``; with ``all_codes``, every
    one of the 254 non-NaN codes (subnormals through +-448) equally likely.
    Codes are drawn directly as bit patterns (no value is quantised here); NaN
    codes never occur.  Chunked and seeded per chunk like ``normal_array``."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint8)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, c))))
        if all_codes:
            r = g.integers(0, 254, size=hi - lo, dtype=np.uint8)        # 0..253
            out[lo:hi] = r + (r >= 0x7F).astype(np.uint8)                # skip 0x7F; 0xFF unreachable
            return
        e = _E4M3_EXP_TABLE[g.integers(0, len(_E4M3_EXP_TABLE), size=hi - lo, dtype=np.uint8)]
        sm = g.integers(0, 16, size=hi - lo, dtype=np.uint8)       # sign bit | 3 mantissa bits
        out[lo:hi] = ((sm & 8) << 4) | (e << 3) | (sm & 7)

    if threads is None:
        threads = min(8, len(os.sched_getaffinity(0)))
    if nchunks <= 1 or threads <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


@dataclass
class Workload:
    """One batch of decode inputs, as raw storage arrays."""
    name: str
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray      # int32 [S]
    block_tables: np.ndarray      # int32 [S][MB], -1 padded
    q: np.ndarray                 # [S][H][D]
    key_cache: np.ndarray         # [NB][Hkv][B][D]
    value_cache: np.ndarray       # [NB][Hkv][B][D]
    new_key: np.ndarray           # [S][Hkv][D]: K of each sequence's newest token
    new_value: np.ndarray         # [S][Hkv][D]
    scale: float
    partition_size: int = 0       # 0: the library picks
    seed: int = 0
    cw_slots: np.ndarray | None = None   # int64 [T]: cache-write timing case
    cw_key: np.ndarray | None = None     # [T][Hkv][D]
    cw_value: np.ndarray | None = None
    notes: dict = field(default_factory=dict)
    kv_dtype: str | None = None   # pool storage type when it differs from dtype ("fp8")
    k_scale: float = 1.0          # fp8 pools: value = code * scale
    v_scale: float = 1.0

    @property
    def pool_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


def _blocks_for(n: int, b: int) -> int:
    """Table width a context of ``n`` tokens occupies (input sizing only)."""
    return -(-n // b)


def _poison_unused(wl_key: np.ndarray, wl_val: np.ndarray, tables: np.ndarray,
                   ctx: np.ndarray, b: int, dtype: str) -> None:
    """NaN every slot that no context covers.  Walks each table by appending
    tokens one block at a time, independent of any slot formula."""
    nb = wl_key.shape[0]
    live = np.zeros((nb, b), dtype=bool)
    for s in range(tables.shape[0]):
        remaining = int(ctx[s])
        j = 0
        while remaining > 0:
            take = min(remaining, b)
            live[tables[s, j], :take] = True
            remaining -= take
            j += 1
    nanw = nan_bits(dtype)
    dead_blocks = ~live.any(axis=1)
    wl_key[dead_blocks] = nanw
    wl_val[dead_blocks] = nanw
    partial = np.nonzero(live.any(axis=1) & ~live.all(axis=1))[0]
    for blk in partial:
        dead = ~live[blk]
        wl_key[blk][:, dead, :] = nanw
        wl_val[blk][:, dead, :] = nanw


def build(name: str, dtype: str, ctx, num_heads: int, num_kv_heads: int, head_dim: int,
          block_size: int, seed: int, pool: str = "permutation", pool_factor: float = 1.0,
          value_scale: float = 1.0, shared_prefix_tokens: int = 0, partition_size: int = 0,
          num_blocks: int | None = None, cw_tokens: int = 0, notes: dict | None = None,
          kv_dtype: str | None = None, kv_scale: float = 1.0, v_scale: float | None = None,
          kv_codes: str = "normal") -> Workload:
    """Assemble a workload from sizes.

    ``pool``: "permutation" -- ids are consecutive slices of a random
    permutation of ``num_blocks`` ids; "choice" -- ids drawn without replacement
    from a pool ``pool_factor`` times the blocks needed.  With
    ``shared_prefix_tokens`` the first ``shared_prefix_tokens / block_size``
    table entries of every sequence hold the same physical ids.  E4M3 pools
    (``kv_dtype="fp8"``): scales ``kv_scale`` for K and ``v_scale`` (default
    ``kv_scale``) for V; ``kv_codes="all"`` draws every non-NaN code equally.
    """
    assert dtype in DTYPES
    ctx = np.asarray(ctx, dtype=np.int32)
    S = int(ctx.shape[0])
    B = block_size
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(0,))))
    per_seq = [_blocks_for(int(c), B) for c in ctx]
    MB = max(per_seq) if S else 1
    MB = max(MB, 1)
    tables = np.full((S, MB), -1, dtype=np.int32)
    if shared_prefix_tokens:
        assert shared_prefix_tokens % B == 0
        nshared = shared_prefix_tokens // B
        private = [n - nshared for n in per_seq]
        assert min(private) >= 0
        needed = nshared + sum(private)
        NB = needed if num_blocks is None else num_blocks
        perm = rng.permutation(NB).astype(np.int32)
        shared_ids = perm[:nshared]
        pos = nshared
        for s in range(S):
            tables[s, :nshared] = shared_ids
            tables[s, nshared:per_seq[s]] = perm[pos:pos + private[s]]
            pos += private[s]
    else:
        needed = sum(per_seq)
        if pool == "choice":
            NB = int(math.ceil(pool_factor * needed)) if num_blocks is None else num_blocks
            ids = rng.choice(NB, needed, replace=False).astype(np.int32)
        else:
            NB = needed if num_blocks is None else num_blocks
            ids = rng.permutation(NB)[:needed].astype(np.int32)
        pos = 0
        for s in range(S):
            tables[s, :per_seq[s]] = ids[pos:pos + per_seq[s]]
            pos += per_seq[s]
    NB = max(NB, 1)
    H, Hkv, D = num_heads, num_kv_heads, head_dim
    q = normal_array(seed, _STREAM["q"], (S, H, D), dtype, value_scale)
    if kv_dtype == "fp8":
        kc = e4m3_codes(seed, _STREAM["k"], (NB, Hkv, B, D), all_codes=kv_codes == "all")
        vc = e4m3_codes(seed, _STREAM["v"], (NB, Hkv, B, D), all_codes=kv_codes == "all")
    else:
        kc = normal_array(seed, _STREAM["k"], (NB, Hkv, B, D), dtype, value_scale)
        vc = normal_array(seed, _STREAM["v"], (NB, Hkv, B, D), dtype, value_scale)
    _poison_unused(kc, vc, tables, ctx, B, kv_dtype or dtype)
    nk = normal_array(seed, _STREAM["new_k"], (S, Hkv, D), dtype, value_scale)
    nv = normal_array(seed, _STREAM["new_v"], (S, Hkv, D), dtype, value_scale)
    wl = Workload(name=name, dtype=dtype, num_seqs=S, num_heads=H, num_kv_heads=Hkv, head_dim=D,
                  block_size=B, num_blocks=NB, context_lens=ctx, block_tables=tables, q=q,
                  key_cache=kc, value_cache=vc, new_key=nk, new_value=nv,
                  scale=1.0 / math.sqrt(D), partition_size=partition_size, seed=seed,
                  notes=dict(notes or {}), kv_dtype=kv_dtype,
                  k_scale=kv_scale if kv_dtype else 1.0,
                  v_scale=(kv_scale if v_scale is None else v_scale) if kv_dtype else 1.0)
    if cw_tokens:
        wl.cw_slots = rng.choice(NB * B, cw_tokens, replace=False).astype(np.int64)
        wl.cw_key = normal_array(seed, _STREAM["cw_k"], (cw_tokens, Hkv, D), dtype, value_scale)
        wl.cw_value = normal_array(seed, _STREAM["cw_v"], (cw_tokens, Hkv, D), dtype, value_scale)
    return wl


# ---------------------------------------------------------------------------
# The five decode workloads.  Shapes follow LLaMA-style layers: 7B (32 heads of
# 128), 13B (40 heads of 128), a 70B-style grouped-query share (64 query heads
# over 8 kv heads) and a 32k-token shared-prefix case.
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    0: "tiny_f32",
    1: "llama7b_f16",
    2: "llama13b_bf16",
    3: "gqa70b_bf16",
    4: "longctx_prefix_f16",
    5: "llama7b_fp8kv",
    6: "gqa70b_fp8kv",
}


def make_workload(index: int, seed: int | None = None, block_size: int | None = None,
                  num_seqs: int | None = None, head_scale: int = 1,
                  ctx_override=None) -> Workload:
    """Workload ``index`` (0..6).  ``seed`` defaults to the index.

    ``num_seqs`` / ``head_scale`` (divide head counts by it) / ``ctx_override``
    shrink a workload for oracle-sized parity runs without changing its
    recipe.
    """
    seed = index if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(99,))))
    name = CONFIG_NAMES[index]
    if index == 0:
        ctx = [17, 50, 128, 200]
        if num_seqs is not None:
            ctx = ctx[:num_seqs]
        if ctx_override is not None:
            ctx = ctx_override
        return build(name, "f32", ctx, 8 // head_scale, 8 // head_scale, 64, block_size or 16, seed,
                     pool="permutation", num_blocks=64 if ctx_override is None else None)
    if index == 1:
        S = num_seqs or 32
        ctx = rng.integers(512, 2048 + 1, size=S) if ctx_override is None else ctx_override
        return build(name, "f16", ctx, 32 // head_scale, 32 // head_scale, 128, block_size or 16, seed,
                     pool="choice", pool_factor=1.2, value_scale=0.5)
    if index == 2:
        S = num_seqs or 64
        ctx = [2048] * S if ctx_override is None else ctx_override
        return build(name, "bf16", ctx, 40 // head_scale, 40 // head_scale, 128, block_size or 16, seed,
                     pool="permutation", cw_tokens=64)
    if index == 3:
        S = num_seqs or 16
        ctx = rng.integers(2048, 4096 + 1, size=S) if ctx_override is None else ctx_override
        return build(name, "bf16", ctx, 64 // head_scale, 8 // head_scale, 128, block_size or 16, seed,
                     pool="permutation")
    if index == 4:
        S = num_seqs or 8
        ctx = [32768] * S if ctx_override is None else ctx_override
        return build(name, "f16", ctx, 32 // head_scale, 32 // head_scale, 128, block_size or 64, seed,
                     pool="permutation", shared_prefix_tokens=2048, partition_size=512)
    if index == 5:
        # The LLaMA-7B-shaped layer with 8-bit (E4M3) K/V pools, scale 0.5:
        # fp16 queries and outputs, random codes in the pools.
        S = num_seqs or 32
        ctx = rng.integers(512, 2048 + 1, size=S) if ctx_override is None else ctx_override
        return build(name, "f16", ctx, 32 // head_scale, 32 // head_scale, 128, block_size or 16, seed,
                     pool="choice", pool_factor=1.2, value_scale=0.5, kv_dtype="fp8",
                     kv_scale=0.5)
    if index == 6:
        # The 70B-style grouped-query share with 8-bit (E4M3) K/V pools, scale
        # 0.5: bf16 queries and outputs over 8 kv heads of 8 query heads each.
        S = num_seqs or 16
        ctx = rng.integers(2048, 4096 + 1, size=S) if ctx_override is None else ctx_override
        return build(name, "bf16", ctx, 64 // head_scale, 8 // head_scale, 128, block_size or 16,
                     seed, pool="permutation", kv_dtype="fp8", kv_scale=0.5)
    raise ValueError(index)


# ---------------------------------------------------------------------------
# Device copies (plumbing only: the raw words are moved, never converted)
# ---------------------------------------------------------------------------

def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "fp8": torch.uint8}[dtype]


def to_torch(raw: np.ndarray, dtype: str, device="cpu"):
    """The raw storage words of ``raw`` as a torch tensor of the storage type
    (fp8 codes as uint8)."""
    import torch
    arr = np.ascontiguousarray(raw)
    if dtype == "bf16":
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    return t.to(device)


def from_torch(t, dtype: str) -> np.ndarray:
    """Raw storage words of a torch tensor as numpy (bf16 as uint16)."""
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclass
class DeviceWorkload:
    q: object
    key_cache: object
    value_cache: object
    block_tables: object
    context_lens: object
    new_key: object
    new_value: object
    out: object


def to_device(wl: Workload, device="cuda") -> DeviceWorkload:
    import torch
    q = to_torch(wl.q, wl.dtype, device)
    return DeviceWorkload(
        q=q,
        key_cache=to_torch(wl.key_cache, wl.pool_dtype, device),
        value_cache=to_torch(wl.value_cache, wl.pool_dtype, device),
        block_tables=torch.from_numpy(wl.block_tables).to(device),
        context_lens=torch.from_numpy(wl.context_lens).to(device),
        new_key=to_torch(wl.new_key, wl.dtype, device),
        new_value=to_torch(wl.new_value, wl.dtype, device),
        out=torch.empty_like(q),
    )


# ---------------------------------------------------------------------------
# Block-manager schedules (host side): the request events a continuous-
# batching decode loop sends to a block manager.  Pure bookkeeping of request
# lengths; nothing here depends on which blocks a manager hands out.
# ---------------------------------------------------------------------------

SYSTEM_PROMPT_ID = 1 << 40


def block_manager_schedule(seed: int, batch: int, steps: int, system_prompt: int = 1024,
                           share_frac: float = 0.25, fork_prob: float = 0.02,
                           prompt=(512, 2048), generate=(32, 256)):
    """Events of ``steps`` decode steps over ``batch`` live requests.

    Returns ``(setup, per_step)``: ``setup`` admits the system prompt and the
    first ``batch`` requests; ``per_step[k]`` is the events of step k.  Events:
      ("alloc", rid, num_tokens)          prompt allocation
      ("share", src, dst, shared_len)     prefix sharing of the system prompt
      ("append", rids, positions)         int64 / int32 arrays, in order
      ("fill", rids)                      the step's block tables for decode
      ("free", rid)                       a finished request
      ("fork", src, dst)                  a beam fork of a live request
    A request's prompt length is uniform in ``prompt``; ``share_frac`` of the
    requests start from the system prompt (shared, then their own tokens
    appended one position at a time); each generates a number of tokens
    uniform in ``generate`` and is then freed and replaced.  Each step every
    live request appends the token at its current length."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(98,))))
    live: dict[int, list[int]] = {}
    next_id = [0]

    def admit(ev):
        rid = next_id[0]
        next_id[0] += 1
        plen = int(rng.integers(prompt[0], prompt[1] + 1))
        if rng.random() < share_frac:
            plen = max(plen, system_prompt)
            ev.append(("share", SYSTEM_PROMPT_ID, rid, system_prompt))
            if plen > system_prompt:
                ev.append(("append", np.full(plen - system_prompt, rid, dtype=np.int64),
                           np.arange(system_prompt, plen, dtype=np.int32)))
        else:
            ev.append(("alloc", rid, plen))
        live[rid] = [plen, int(rng.integers(generate[0], generate[1] + 1))]

    setup = [("alloc", SYSTEM_PROMPT_ID, system_prompt)]
    for _ in range(batch):
        admit(setup)
    per_step = []
    for _ in range(steps):
        ev = []
        rids = np.fromiter(live.keys(), dtype=np.int64, count=len(live))
        pos = np.array([live[int(r)][0] for r in rids], dtype=np.int32)
        ev.append(("append", rids, pos))
        ev.append(("fill", rids))
        done = []
        for r in rids:
            st = live[int(r)]
            st[0] += 1
            st[1] -= 1
            if st[1] <= 0:
                done.append(int(r))
        for r in done:
            ev.append(("free", r))
            del live[r]
            admit(ev)
        if rng.random() < fork_prob * len(live) / max(batch, 1):
            src = int(rids[int(rng.integers(len(rids)))])
            if src in live:
                dst = next_id[0]
                next_id[0] += 1
                ev.append(("fork", src, dst))
                live[dst] = [live[src][0], int(rng.integers(generate[0], generate[1] + 1))]
        per_step.append(ev)
    return setup, per_step
