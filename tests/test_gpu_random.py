"""GPU parity over seeded random shapes: every decode entry point (pa_decode,
pa_append_decode and their E4M3 forms) against the oracle on a spread of
dtypes, head dims, block sizes, head groupings (vector and matrix-core
kernels, and groupings above 16 that fall back to the vector kernel),
context lengths (zero, one, block edges, a few thousand) and partition
sizes.  The cases are drawn from a fixed seed, so every run tests the same
ones; each prints its parameters before it runs.

Bars as in the other parity tests: pools bit-exact after an appending call,
outputs within the decode tolerance."""
import sys

import numpy as np
import pytest
import torch

import oracle.paged as P
import tests._bounds as BD
import paged_kv_cache_368_amd as pa
from workloads import build, from_torch, nan_bits, to_device

pytestmark = pytest.mark.gpu

NUM_CASES = 32


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    kind = ["decode", "append", "decode_fp8", "append_fp8"][i % 4]
    fp8 = kind.endswith("fp8")
    dtype = str(rng.choice(["f16", "bf16"] if fp8 else ["f32", "f16", "bf16"]))
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([16, 32, 64]))
    Hkv = int(rng.choice([1, 2, 3]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 17]))
    S = int(rng.integers(1, 6))
    edges = [0, 1, B - 1, B, B + 1, 2 * B]
    ctx = [int(rng.choice(edges)) if rng.random() < 0.4 else int(rng.integers(2, 2500))
           for _ in range(S)]
    step = max(B, 16)
    ps = 0 if rng.random() < 0.4 else step * int(rng.integers(1, 1024 // step + 1))
    return dict(kind=kind, dtype=dtype, D=D, B=B, H=Hkv * G, Hkv=Hkv, ctx=ctx, ps=ps,
                seed=2000 + i)


CASES = [_draw(i) for i in range(NUM_CASES)]


@pytest.mark.parametrize("case", CASES, ids=[f"{c['kind']}-{i}" for i, c in enumerate(CASES)])
def test_random_shapes(case):
    c = case
    _say(" ".join(f"{k}={v}" for k, v in c.items()))
    fp8 = c["kind"].endswith("fp8")
    wl = build("random", c["dtype"], c["ctx"], c["H"], c["Hkv"], c["D"], c["B"],
               seed=c["seed"], pool="choice", pool_factor=1.3,
               kv_dtype="fp8" if fp8 else None, kv_scale=0.375)
    kc, vc = wl.key_cache.copy(), wl.value_cache.copy()
    if c["kind"].startswith("append"):
        slots = P.compute_slots(wl.block_tables, wl.block_size, wl.num_blocks,
                                context_lens=wl.context_lens)
        for sl in slots:                  # the slot's old contents must never count
            if sl >= 0:
                b, off = divmod(int(sl), wl.block_size)
                wl.key_cache[b, :, off, :] = 0x7F if fp8 else nan_bits(wl.dtype)
                wl.value_cache[b, :, off, :] = 0xFF if fp8 else nan_bits(wl.dtype)
        kc, vc = wl.key_cache.copy(), wl.value_cache.copy()
        if fp8:
            P.cache_write_fp8(kc, vc, wl.new_key, wl.new_value, slots, wl.block_size, wl.dtype,
                              wl.k_scale, wl.v_scale)
        else:
            P.cache_write(kc, vc, wl.new_key, wl.new_value, slots, wl.block_size)
    if fp8:
        ref = P.paged_decode_fp8(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.block_size,
                                 wl.scale, wl.dtype, wl.k_scale, wl.v_scale, wl.num_kv_heads)
    else:
        ref = P.paged_decode(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.block_size,
                             wl.scale, wl.dtype, wl.num_kv_heads)

    dev = to_device(wl)
    mctx = max(int(wl.context_lens.max()), 1)
    if c["kind"] == "decode":
        pa.pa_decode(dev.out, dev.q, dev.key_cache, dev.value_cache, dev.block_tables,
                     dev.context_lens, mctx, wl.scale, c["ps"],
                     workspace=pa.decode_workspace(dev.q, dev.key_cache, mctx, c["ps"]))
    elif c["kind"] == "append":
        pa.pa_append_decode(dev.out, dev.q, dev.new_key, dev.new_value, dev.key_cache,
                            dev.value_cache, dev.block_tables, dev.context_lens, mctx, wl.scale,
                            c["ps"],
                            workspace=pa.decode_workspace(dev.q, dev.key_cache, mctx, c["ps"]))
    elif c["kind"] == "decode_fp8":
        pa.pa_decode_fp8(dev.out, dev.q, dev.key_cache, dev.value_cache, dev.block_tables,
                         dev.context_lens, mctx, wl.k_scale, wl.v_scale, wl.scale, c["ps"],
                         workspace=pa.decode_workspace(dev.q, dev.key_cache, mctx, c["ps"]))
    else:
        pa.pa_append_decode_fp8(dev.out, dev.q, dev.new_key, dev.new_value, dev.key_cache,
                                dev.value_cache, dev.block_tables, dev.context_lens, mctx,
                                wl.k_scale, wl.v_scale, wl.scale, c["ps"],
                                workspace=pa.decode_workspace(dev.q, dev.key_cache, mctx, c["ps"]))
    torch.cuda.synchronize()
    got = P.to_f64(from_torch(dev.out, wl.dtype), wl.dtype)
    BD.assert_close(got, ref, wl.dtype, c["kind"])
    pool_dt = "fp8" if fp8 else wl.dtype
    assert np.array_equal(from_torch(dev.key_cache, pool_dt).view(np.uint8),
                          kc.view(np.uint8)), "K pool"
    assert np.array_equal(from_torch(dev.value_cache, pool_dt).view(np.uint8),
                          vc.view(np.uint8)), "V pool"
