"""GPU parity of split-context decode when one vector work-group streams
several consecutive partitions of a (sequence, head).

The vector decode launch gives a work-group four consecutive partitions (each
still written as its own partial and merged by log-sum-exp, P2 section 4.1's
split-and-merge with P1 section 7's merge) when the context is split at least
eight ways and the launch still has at least 4096 work-groups after the
grouping.  The shapes here (32 sequences x 32 heads, contexts up to 2048
tokens in partitions of 64, 80 or 128 tokens) are sized to take that path;
partitions of 256 tokens (eight of them, 2048 work-groups once grouped) stay
one per work-group and serve as the control.  Ragged contexts leave groups
with fewer than four partitions, or none, and partitions of 80 tokens give
the waves of a work-group unequal chunk counts.

Bars: outputs within the decode tolerance of the float64 oracle (2e-3 for
fp16/bf16, per element at least one unit of the output's last place), pools
bit-exact after appending, invalid table entries or contexts poisoning
exactly their own sequence's rows.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.paged as P
import tests._bounds as BD
import paged_kv_cache_368_amd as pa
from workloads import build, from_torch, nan_bits, to_device

pytestmark = pytest.mark.gpu

S, H, B = 32, 32, 16


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()


def _contexts(seed):
    """Ragged contexts, the longest exactly 2048; a few short ones whose
    sequences leave most partition groups empty."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(900, 2049, size=S)
    ctx[0] = 2048
    ctx[1], ctx[2], ctx[3] = 1, 17, 130
    ctx[4] = 1280                     # exactly ten partitions of 128
    return ctx


def _workload(dtype, D, seed, kv=None):
    return build("groups", dtype, _contexts(seed), H, H, D, B, seed=seed, pool="choice",
                 pool_factor=1.2, kv_dtype=kv, kv_scale=0.5 if kv else 1.0)


def _workspace(dev, maxctx, ps):
    ws = pa.decode_workspace(dev.q, dev.key_cache, maxctx, ps)
    assert ws is not None
    ws.fill_(255)                     # NaN partials: every one read must have been written
    return ws


def _oracle(wl):
    if wl.kv_dtype == "fp8":
        return P.paged_decode_fp8(wl.q, wl.key_cache, wl.value_cache, wl.block_tables,
                                  wl.context_lens, wl.block_size, wl.scale, wl.dtype,
                                  wl.k_scale, wl.v_scale, wl.num_kv_heads)
    return P.paged_decode(wl.q, wl.key_cache, wl.value_cache, wl.block_tables, wl.context_lens,
                          wl.block_size, wl.scale, wl.dtype, wl.num_kv_heads)


def _decode(wl, dev, ps, maxctx=None):
    maxctx = maxctx or wl.max_context_len
    ws = _workspace(dev, maxctx, ps)
    if wl.kv_dtype == "fp8":
        pa.pa_decode_fp8(dev.out, dev.q, dev.key_cache, dev.value_cache, dev.block_tables,
                         dev.context_lens, maxctx, wl.k_scale, wl.v_scale, wl.scale, ps,
                         workspace=ws)
    else:
        pa.pa_decode(dev.out, dev.q, dev.key_cache, dev.value_cache, dev.block_tables,
                     dev.context_lens, maxctx, wl.scale, ps, workspace=ws)
    torch.cuda.synchronize()
    return P.to_f64(from_torch(dev.out, wl.dtype), wl.dtype)


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128)])
def test_groups_decode(dtype, D):
    wl = _workload(dtype, D, seed=300 + D)
    ref = _oracle(wl)
    dev = to_device(wl)
    for ps in (64, 80, 128, 256):
        _say(f"groups decode {dtype} D={D} P={ps}")
        BD.assert_close(_decode(wl, dev, ps), ref, dtype, f"groups {dtype} D={D} P={ps}")


def test_groups_decode_fp8():
    wl = _workload("f16", 128, seed=311, kv="fp8")
    ref = _oracle(wl)
    dev = to_device(wl)
    for ps in (80, 128):
        _say(f"groups decode fp8 P={ps}")
        BD.assert_close(_decode(wl, dev, ps), ref, "f16", f"groups fp8 P={ps}")


@pytest.mark.parametrize("ps", [80, 128])
def test_groups_append(ps):
    """The one-launch step: the newest token's slot holds NaN before the
    call, so an output that read the slot instead of the input row shows."""
    _say(f"groups append P={ps}")
    wl = _workload("bf16", 128, seed=320 + ps)
    slots = P.compute_slots(wl.block_tables, wl.block_size, wl.num_blocks,
                            context_lens=wl.context_lens)
    for sl in slots:
        b, off = divmod(int(sl), wl.block_size)
        wl.key_cache[b, :, off, :] = nan_bits(wl.dtype)
        wl.value_cache[b, :, off, :] = nan_bits(wl.dtype)
    kc, vc = wl.key_cache.copy(), wl.value_cache.copy()
    P.cache_write(kc, vc, wl.new_key, wl.new_value, slots, wl.block_size)
    ref = P.paged_decode(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.block_size,
                         wl.scale, wl.dtype, wl.num_kv_heads)
    dev = to_device(wl)
    pa.pa_append_decode(dev.out, dev.q, dev.new_key, dev.new_value, dev.key_cache,
                        dev.value_cache, dev.block_tables, dev.context_lens, wl.max_context_len,
                        wl.scale, ps, workspace=_workspace(dev, wl.max_context_len, ps))
    torch.cuda.synchronize()
    got = P.to_f64(from_torch(dev.out, wl.dtype), wl.dtype)
    BD.assert_close(got, ref, wl.dtype, f"groups append P={ps}")
    assert from_torch(dev.key_cache, wl.dtype).tobytes() == kc.tobytes(), "K pool"
    assert from_torch(dev.value_cache, wl.dtype).tobytes() == vc.tobytes(), "V pool"


def test_groups_invalid_values_poison_only_their_rows():
    """A block id outside the pool in the third partition of a group, a
    negative one in the second partition of another group, and a context
    beyond the maximum: NaN in exactly those sequences' rows."""
    _say("groups poison")
    wl = _workload("f16", 128, seed=330)
    ref = _oracle(wl)
    ps = 128
    assert wl.context_lens[5] > 3 * ps and wl.context_lens[6] > 6 * ps
    wl.block_tables[5, (2 * ps) // B + 3] = wl.num_blocks + 3     # partition 2 (group 0)
    wl.block_tables[6, (5 * ps) // B + 1] = -5                    # partition 5 (group 1)
    wl.context_lens[7] = 4096                                     # beyond max_context_len
    dev = to_device(wl)
    got = _decode(wl, dev, ps, maxctx=2048)
    for s in (5, 6, 7):
        assert np.isnan(got[s]).all(), f"sequence {s} not poisoned: {got[s, :2, :4]}"
    healthy = [s for s in range(S) if s not in (5, 6, 7)]
    BD.assert_close(got[healthy], ref[healthy], "f16", "groups healthy rows")
