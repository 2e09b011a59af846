"""GPU: decode steps recorded in a HIP graph replay to the same bytes as the
eager calls.

A serving loop records the step once and replays it every token.  The
library allocates nothing inside a call and issues no memset or
synchronisation, so the whole step (one launch, or slots + cache write +
attention, with the merge of split contexts) can be recorded through
``torch.cuda.graph`` on the binding's current stream.  Each case runs the
step eagerly (checked against the float64 oracle), records it, then replays
it several times with the program's own eager work and synchronisations
between the replays, after poisoning the output each time, and compares
every replay with the eager call bit for bit (the same kernels on the same
inputs).  The appended rows go to the same slots on every replay, so the
pools must come out byte-equal too.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.paged as P
import tests._bounds as B
import paged_kv_cache_368_amd as pa
from workloads import build, from_torch, to_device

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()


def _workload(name, dtype, H, Hkv, kv, ps):
    ctx = np.random.default_rng(77).integers(600, 3000, size=4)
    return build(f"graph_{name}", dtype, ctx, H, Hkv, 128, 16, seed=77, partition_size=ps,
                 kv_dtype=kv, kv_scale=0.5 if kv else 1.0)


def _oracle_after_append(wl):
    """Attention over the pools once each sequence's newest token is written."""
    slots = P.compute_slots(wl.block_tables, wl.block_size, wl.num_blocks,
                            context_lens=wl.context_lens)
    kc, vc = wl.key_cache.copy(), wl.value_cache.copy()
    if wl.pool_dtype == "fp8":
        P.cache_write_fp8(kc, vc, wl.new_key, wl.new_value, slots, wl.block_size, wl.dtype,
                          wl.k_scale, wl.v_scale)
        return P.paged_decode_fp8(wl.q, kc, vc, wl.block_tables, wl.context_lens,
                                  wl.block_size, wl.scale, wl.dtype, wl.k_scale, wl.v_scale,
                                  wl.num_kv_heads)
    P.cache_write(kc, vc, wl.new_key, wl.new_value, slots, wl.block_size)
    return P.paged_decode(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.block_size,
                          wl.scale, wl.dtype, wl.num_kv_heads)


def _replay_matches(step, dev, what):
    """Eager step, then REPLAYS graph replays: every replay byte-equal to it."""
    step()
    torch.cuda.synchronize()
    want = (dev.out.clone(), dev.key_cache.clone(), dev.value_cache.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    noise = torch.empty(1 << 20, device="cuda")
    for i in range(REPLAYS):
        dev.out.fill_(float("nan"))                 # a replay that skips the output shows
        noise.normal_()
        float(noise.sum())                          # eager work and a sync between replays
        g.replay()
        torch.cuda.synchronize()
        for got, ref, name in zip((dev.out, dev.key_cache, dev.value_cache), want,
                                  ("out", "key_cache", "value_cache")):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), \
                f"{what}: replay {i}: {name} differs from the eager call"
    return want[0]


# (name, query dtype, H, Hkv, pool type, partition length): the vector kernel
# and the matrix-core kernel, split (merge launch) and not.
CASES = [("mha_f16_split", "f16", 8, 8, None, 512),
         ("mha_bf16_whole", "bf16", 8, 8, None, 4096),
         ("gqa_bf16_split", "bf16", 16, 2, None, 512),
         ("gqa_f16_fp8_split", "f16", 16, 2, "fp8", 512)]


@pytest.mark.parametrize("name,dtype,H,Hkv,kv,ps", CASES, ids=[c[0] for c in CASES])
def test_graph_one_launch_step(name, dtype, H, Hkv, kv, ps):
    _say(f"graph append decode {name}")
    wl = _workload(name, dtype, H, Hkv, kv, ps)
    dev = to_device(wl)
    ws = pa.decode_workspace(dev.q, dev.key_cache, wl.max_context_len, ps)
    if kv:
        def step():
            pa.pa_append_decode_fp8(dev.out, dev.q, dev.new_key, dev.new_value, dev.key_cache,
                                    dev.value_cache, dev.block_tables, dev.context_lens,
                                    wl.max_context_len, wl.k_scale, wl.v_scale, wl.scale, ps,
                                    workspace=ws)
    else:
        def step():
            pa.pa_append_decode(dev.out, dev.q, dev.new_key, dev.new_value, dev.key_cache,
                                dev.value_cache, dev.block_tables, dev.context_lens,
                                wl.max_context_len, wl.scale, ps, workspace=ws)
    out = _replay_matches(step, dev, name)
    B.assert_close(P.to_f64(from_torch(out, wl.dtype), wl.dtype), _oracle_after_append(wl),
                   wl.dtype, f"graph {name}")


def test_graph_three_call_step():
    """Slots, cache write and the split decode with its merge, as one graph."""
    _say("graph three-call step")
    wl = _workload("three_call", "bf16", 16, 2, None, 512)
    dev = to_device(wl)
    ps = wl.partition_size
    ws = pa.decode_workspace(dev.q, dev.key_cache, wl.max_context_len, ps)
    slots = torch.empty(wl.num_seqs, dtype=torch.int64, device="cuda")

    def step():
        pa.pa_compute_slots(slots, dev.block_tables, wl.block_size, wl.num_blocks,
                            context_lens=dev.context_lens)
        pa.pa_cache_write(dev.new_key, dev.new_value, dev.key_cache, dev.value_cache, slots)
        pa.pa_decode(dev.out, dev.q, dev.key_cache, dev.value_cache, dev.block_tables,
                     dev.context_lens, wl.max_context_len, wl.scale, ps, workspace=ws)
    out = _replay_matches(step, dev, "three-call step")
    B.assert_close(P.to_f64(from_torch(out, wl.dtype), wl.dtype), _oracle_after_append(wl),
                   wl.dtype, "graph three-call step")


def test_graph_noalloc_decode():
    """The workspace-free entry point records too (its scratch address is
    taken on the first, eager, call)."""
    _say("graph no-alloc decode")
    wl = _workload("noalloc", "f16", 8, 8, None, 512)
    dev = to_device(wl)

    def step():
        pa.pa_decode_noalloc(dev.out, dev.q, dev.key_cache, dev.value_cache, dev.block_tables,
                             dev.context_lens, wl.max_context_len, wl.scale, wl.partition_size)
    out = _replay_matches(step, dev, "no-alloc decode")
    ref = P.paged_decode(wl.q, wl.key_cache, wl.value_cache, wl.block_tables, wl.context_lens,
                         wl.block_size, wl.scale, wl.dtype, wl.num_kv_heads)
    B.assert_close(P.to_f64(from_torch(out, wl.dtype), wl.dtype), ref, wl.dtype,
                   "graph no-alloc decode")
