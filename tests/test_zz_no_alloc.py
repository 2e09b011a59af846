"""GPU check of pa_decode_noalloc, the decode entry point that takes no
workspace (its split-context partials live in the library's static per-GPU
scratch): on two calls in a row, the second smaller, its output equals
pa_decode's with a caller workspace bit for bit and the float64 oracle
within the decode bars.  The first call also runs on the vector kernel and
the matrix-core grouped-query kernel."""
import sys

import numpy as np
import pytest
import torch

import oracle.paged as P
import tests._bounds as BD
import paged_kv_cache_368_amd as pa
from workloads import from_torch, make_workload, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()


def _both(wl, ps):
    """(pa_decode_noalloc output, pa_decode output) as raw storage words."""
    dev = to_device(wl)
    need = pa.pa_decode_workspace_size(wl.num_seqs, wl.num_heads, wl.num_kv_heads, wl.head_dim,
                                       wl.block_size, wl.max_context_len, ps, dev.q.dtype)
    assert 0 < need <= pa.PA_NOALLOC_SCRATCH_BYTES, "the case must use the scratch"
    out_ref = torch.empty_like(dev.out)
    # the reference call first: its workspace holds other partials than the scratch
    pa.pa_decode(out_ref, dev.q, dev.key_cache, dev.value_cache, dev.block_tables,
                 dev.context_lens, wl.max_context_len, wl.scale, ps,
                 workspace=pa.decode_workspace(dev.q, dev.key_cache, wl.max_context_len, ps))
    pa.pa_decode_noalloc(dev.out, dev.q, dev.key_cache, dev.value_cache, dev.block_tables,
                         dev.context_lens, wl.max_context_len, wl.scale, ps)
    torch.cuda.synchronize()
    return from_torch(dev.out, wl.dtype), from_torch(out_ref, wl.dtype)


def _check(wl, ps, what):
    got, ref = _both(wl, ps)
    assert got.tobytes() == ref.tobytes(), f"{what}: differs from pa_decode"
    exp = P.paged_decode(wl.q, wl.key_cache, wl.value_cache, wl.block_tables, wl.context_lens,
                         wl.block_size, wl.scale, wl.dtype, wl.num_kv_heads)
    BD.assert_close(P.to_f64(got, wl.dtype), exp, wl.dtype, what)


@pytest.mark.parametrize("index,first,second,ps", [
    # long-context shape (vector kernel), fp16, P = 512; then fewer, shorter sequences
    (4, dict(num_seqs=3, head_scale=4, ctx_override=[4096, 2600, 3333]),
     dict(num_seqs=2, head_scale=8, ctx_override=[2600, 2100]), 512),
    # 70B-style grouped-query share (matrix cores), bf16, P = 256; then a smaller one
    (3, dict(num_seqs=4, head_scale=2, ctx_override=[2048, 3000, 1111, 2500]),
     dict(num_seqs=2, head_scale=4, ctx_override=[900, 257]), 256),
])
def test_noalloc_matches_decode_on_two_calls(index, first, second, ps):
    _say(f"noalloc workload {index} first call")
    _check(make_workload(index, **first), ps, f"workload {index}, first call")
    _say(f"noalloc workload {index} second (smaller) call")
    _check(make_workload(index, **second), ps, f"workload {index}, second call")


def test_noalloc_without_a_split_needs_no_scratch():
    _say("noalloc single partition")
    wl = make_workload(1, num_seqs=3, head_scale=8, ctx_override=[700, 64, 1000])
    dev = to_device(wl)
    pa.pa_decode_noalloc(dev.out, dev.q, dev.key_cache, dev.value_cache, dev.block_tables,
                         dev.context_lens, wl.max_context_len, wl.scale, 0)
    torch.cuda.synchronize()
    exp = P.paged_decode(wl.q, wl.key_cache, wl.value_cache, wl.block_tables, wl.context_lens,
                         wl.block_size, wl.scale, wl.dtype, wl.num_kv_heads)
    BD.assert_close(P.to_f64(from_torch(dev.out, wl.dtype), wl.dtype), exp, wl.dtype,
                    "single partition")
    assert np.isfinite(P.to_f64(from_torch(dev.out, wl.dtype), wl.dtype)).all()
