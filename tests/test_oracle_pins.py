"""CPU pins of the float64 oracle against facts the pages and mathematics fix.

Every pin here is a plain function without fixtures, so that
``test_oracle_mutations.py`` can re-run them against oracles with planted
mistakes.  Sources P1-P3 are as in the ``oracle`` package docstring.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle.paged as P
import tests._fp8_cases as FP8C
from workloads import build, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _place(kc, vc, contig_k, contig_v, table, block_size):
    """Test-side placement of a contiguous [n][Hkv][D] context into a pool:
    fill the current block slot by slot and move to the next table entry when
    it is full (the append order of P3 section 3); no division is used."""
    j, off = 0, 0
    for t in range(contig_k.shape[0]):
        kc[table[j], :, off, :] = contig_k[t]
        vc[table[j], :, off, :] = contig_v[t]
        off += 1
        if off == block_size:
            j, off = j + 1, 0


# --------------------------------------------------------------------------
# Slot arithmetic
# --------------------------------------------------------------------------

def test_pin_block_counts_page3():
    g = _golden("p3_block_arithmetic.json")
    for tokens, blocks in g["blocks_for_tokens"]:
        assert P.num_required_blocks(tokens, g["block_size"]) == blocks


def test_pin_token17_page3():
    g = _golden("p3_block_arithmetic.json")
    table = [41, 7, 13, 2]
    phys, off = P.physical_location(table, 17, g["block_size"])
    assert (phys, off) == (table[g["token_17"]["logical_block"]], g["token_17"]["offset"])
    assert P.slot_of(table, 17, 16) == 7 * 16 + 1


def test_pin_logical_to_physical_page2():
    g = _golden("p2_logical_to_physical.json")
    names = g["table"]
    ids = [10, 3, 7]                     # arbitrary physical ids standing for A, B, C
    for t, (name, off) in enumerate(g["expected"]):
        phys, o = P.physical_location(ids, t, g["block_size"])
        assert names[ids.index(phys)] == name and o == off
    assert P.physical_location(ids, 12, g["block_size"]) is None   # past the table


def test_pin_slots_brute_force():
    """Slots by division equal slots found by simulating appends token by
    token (a new block is opened exactly when the current one is full)."""
    rng = _rng(1)
    for B in (1, 4, 16, 64):
        for n in (0, 1, B - 1 if B > 1 else 1, B, B + 1, 5 * B + 3):
            nb = P.num_required_blocks(n, B)
            table = rng.permutation(max(nb, 1) * 3)[:nb]
            expected, j, off = [], 0, 0
            for t in range(n):
                expected.append(int(table[j]) * B + off)
                off += 1
                if off == B:
                    j, off = j + 1, 0
            assert [P.slot_of(table, t, B) for t in range(n)] == expected
            assert len(table) == (j + (off > 0))


def test_pin_compute_slots_edges():
    tables = np.array([[5, 2, -1], [7, 1, 3]], dtype=np.int32)
    ctx = np.array([17, 48], dtype=np.int32)
    # newest token of each sequence: position ctx-1
    assert P.compute_slots(tables, 16, 8, context_lens=ctx).tolist() == [2 * 16 + 0, 3 * 16 + 15]
    # explicit positions, invalid cases -> -1: negative, past the table, padding, id out of pool
    got = P.compute_slots(tables, 16, 6, seq_ids=[0, 0, 0, 1, 1, 0],
                          positions=[-1, 48, 33, 0, 20, 3]).tolist()
    assert got == [-1, -1, -1, -1, 1 * 16 + 4, 5 * 16 + 3]
    assert P.compute_slots(tables, 16, 8, context_lens=np.array([0, 1])).tolist() == [-1, 7 * 16]


# --------------------------------------------------------------------------
# Cache write
# --------------------------------------------------------------------------

def test_pin_cache_write_roundtrip_and_sentinels():
    rng = _rng(2)
    for dtype, store in (("f32", np.float32), ("f16", np.float16), ("bf16", np.uint16)):
        NB, Hkv, B, D = 6, 3, 16, 8
        if store is np.uint16:
            kc = rng.integers(0, 1 << 16, size=(NB, Hkv, B, D), dtype=np.uint16)
        else:
            kc = rng.standard_normal((NB, Hkv, B, D)).astype(store)
        vc = kc.copy()
        vc.view(np.uint8)[...] ^= 0x5A
        k0, v0 = kc.copy(), vc.copy()
        T = 10
        slots = rng.choice(NB * B, T, replace=False).astype(np.int64)
        slots[3] = -1                       # padding token: skipped
        slots[7] = NB * B + 5               # outside the pool: skipped
        key = rng.standard_normal((T, Hkv, D)).astype(np.float32).astype(store) if store is not np.uint16 \
            else rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
        val = key[::-1].copy()
        P.cache_write(kc, vc, key, val, slots, B)
        touched = np.zeros((NB, B), bool)
        for i, sl in enumerate(slots):
            if 0 <= sl < NB * B:
                blk, off = divmod(int(sl), B)
                touched[blk, off] = True
                assert kc[blk, :, off, :].tobytes() == key[i].tobytes()
                assert vc[blk, :, off, :].tobytes() == val[i].tobytes()
        for blk in range(NB):
            for off in range(B):
                if not touched[blk, off]:
                    assert kc[blk, :, off].tobytes() == k0[blk, :, off].tobytes()
                    assert vc[blk, :, off].tobytes() == v0[blk, :, off].tobytes()


def test_pin_cache_write_then_gather_is_identity():
    """Appending a whole context token by token through the slot mapping and
    gathering it back through the table returns the context."""
    rng = _rng(3)
    B, Hkv, D, n = 16, 2, 4, 53
    nb = P.num_required_blocks(n, B)
    table = rng.permutation(10)[:nb].astype(np.int32)
    kc = np.zeros((10, Hkv, B, D))
    vc = np.zeros((10, Hkv, B, D))
    K = rng.standard_normal((n, Hkv, D))
    V = rng.standard_normal((n, Hkv, D))
    slots = P.compute_slots(table[None, :], B, 10, seq_ids=[0] * n, positions=list(range(n)))
    P.cache_write(kc, vc, K, V, slots, B)
    for g in range(Hkv):
        np.testing.assert_array_equal(P.gather_context(kc, table, n, g, B), K[:, g])
        np.testing.assert_array_equal(P.gather_context(vc, table, n, g, B), V[:, g])


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _paged_case(rng, S, H, Hkv, D, B, ctx):
    """Contiguous K/V per sequence, placed into a shuffled NaN-filled pool."""
    nbs = [P.num_required_blocks(n, B) for n in ctx]
    NB = sum(nbs) + 3
    perm = rng.permutation(NB)
    tables = np.full((S, max(max(nbs), 1)), -1, dtype=np.int32)
    kc = np.full((NB, Hkv, B, D), np.nan)
    vc = np.full((NB, Hkv, B, D), np.nan)
    contig, pos = [], 0
    for s in range(S):
        tables[s, :nbs[s]] = perm[pos:pos + nbs[s]]
        pos += nbs[s]
        K = rng.standard_normal((ctx[s], Hkv, D))
        V = rng.standard_normal((ctx[s], Hkv, D))
        _place(kc, vc, K, V, tables[s], B)
        contig.append((K, V))
    q = rng.standard_normal((S, H, D))
    return q, kc, vc, tables, np.array(ctx, dtype=np.int32), contig


def test_pin_paged_equals_sdpa_on_contiguous():
    """Library routine: torch's scaled_dot_product_attention in float64 over
    the contiguous context equals the oracle's paged result (P3 section 2:
    paging changes where K/V live, not what attention computes)."""
    rng = _rng(4)
    for (H, Hkv) in ((4, 4), (8, 2)):
        S, D, B = 3, 16, 16
        ctx = [1, 37, 70]
        q, kc, vc, tables, cl, contig = _paged_case(rng, S, H, Hkv, D, B, ctx)
        scale = 1.0 / math.sqrt(D)
        got = _paged_decode64(q, kc, vc, tables, cl, B, scale, Hkv)
        for s in range(S):
            K, V = contig[s]
            kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(H // Hkv, dim=0)[None]
            vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(H // Hkv, dim=0)[None]
            qt = torch.from_numpy(q[s])[None, :, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(),
                                                                   scale=scale)[0, :, 0, :].numpy()
            np.testing.assert_allclose(got[s], ref, rtol=0, atol=1e-13)


def _paged_decode64(q, kc, vc, tables, ctx, B, scale, Hkv):
    """Oracle decode on float64 pools (the f32 storage path, widened)."""
    S, H, D = q.shape
    out = np.zeros((S, H, D))
    for s in range(S):
        for h in range(H):
            out[s, h] = P.decode_one(q[s, h], kc, vc, tables[s], int(ctx[s]),
                                     P.kv_head_of(h, H, Hkv), B, scale)
    return out


def test_pin_permutation_invariance():
    """Relabelling physical blocks (moving the tiles and the table entries
    together) leaves the result bit-identical."""
    wl = make_workload(0)
    out0 = P.paged_decode(wl.q, wl.key_cache, wl.value_cache, wl.block_tables, wl.context_lens,
                          wl.block_size, wl.scale, wl.dtype)
    pi = _rng(5).permutation(wl.num_blocks)
    kc = np.empty_like(wl.key_cache)
    vc = np.empty_like(wl.value_cache)
    kc[pi] = wl.key_cache
    vc[pi] = wl.value_cache
    tables = np.where(wl.block_tables >= 0, pi[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
    out1 = P.paged_decode(wl.q, kc, vc, tables, wl.context_lens, wl.block_size, wl.scale, wl.dtype)
    assert np.array_equal(out0, out1)


def test_pin_context_one_returns_v():
    rng = _rng(6)
    q, kc, vc, tables, cl, contig = _paged_case(rng, 2, 4, 4, 8, 16, [1, 1])
    out = _paged_decode64(q, kc, vc, tables, cl, 16, 0.3, 4)
    for s in range(2):
        assert np.array_equal(out[s], contig[s][1][0])


def test_pin_identical_keys_and_zero_query_give_mean_v():
    rng = _rng(7)
    D, n = 8, 45
    V = rng.standard_normal((n, D))
    K = np.tile(rng.standard_normal(D), (n, 1))
    q = rng.standard_normal(D)
    np.testing.assert_allclose(P.attention(q, K, V, 0.7), V.mean(axis=0), rtol=0, atol=1e-14)
    K2 = rng.standard_normal((n, D))
    np.testing.assert_allclose(P.attention(np.zeros(D), K2, V, 0.7), V.mean(axis=0), rtol=0, atol=1e-14)


def test_pin_two_tokens_closed_form():
    """Two tokens: the weight of token 1 is the logistic function of the
    score difference."""
    rng = _rng(8)
    for _ in range(20):
        D = 5
        q, K, V = rng.standard_normal(D), rng.standard_normal((2, D)), rng.standard_normal((2, D))
        scale = 0.4
        d = scale * (q @ K[1] - q @ K[0])
        w1 = 1.0 / (1.0 + math.exp(-d))
        np.testing.assert_allclose(P.attention(q, K, V, scale), w1 * V[1] + (1 - w1) * V[0],
                                   rtol=0, atol=1e-14)


def test_pin_decimal_brute_force():
    """50-digit decimal evaluation of the softmax-weighted sum on tiny paged
    inputs (S<=2, H<=2, D<=4, n<=2B)."""
    getcontext().prec = 50
    rng = _rng(9)
    B = 4
    q, kc, vc, tables, cl, contig = _paged_case(rng, 2, 2, 1, 4, B, [5, 8])
    scale = 0.5
    out = _paged_decode64(q, kc, vc, tables, cl, B, scale, 1)
    for s in range(2):
        K, V = contig[s]
        for h in range(2):
            sc = [Decimal(scale) * sum(Decimal(float(q[s, h, d])) * Decimal(float(K[t, 0, d]))
                                       for d in range(4)) for t in range(cl[s])]
            m = max(sc)
            w = [(x - m).exp() for x in sc]
            den = sum(w)
            for d in range(4):
                num = sum(w[t] * Decimal(float(V[t, 0, d])) for t in range(cl[s]))
                assert abs(float(num / den) - out[s, h, d]) <= 1e-14


def test_pin_linear_in_v_and_convex():
    rng = _rng(10)
    n, D = 33, 6
    q, K = rng.standard_normal(D), rng.standard_normal((n, D))
    V1, V2 = rng.standard_normal((n, D)), rng.standard_normal((n, D))
    a, b = 0.75, -2.5
    np.testing.assert_allclose(P.attention(q, K, a * V1 + b * V2, 0.3),
                               a * P.attention(q, K, V1, 0.3) + b * P.attention(q, K, V2, 0.3),
                               rtol=0, atol=1e-13)
    o = P.attention(q, K, V1, 0.3)
    assert np.all(o <= V1.max(axis=0) + 1e-15) and np.all(o >= V1.min(axis=0) - 1e-15)


def test_pin_blockwise_sum_is_a_different_quantity():
    """P1 section 1's per-block sum equals attention for one block, not for
    more (the full softmax of its first formula is what decode computes)."""
    rng = _rng(11)
    D, B = 8, 16
    for n, same in ((1, True), (B - 1, True), (B, True), (B + 1, False), (3 * B, False)):
        q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
        a = P.attention(q, K, V, 0.35)
        b = P.blockwise_softmax_sum(q, K, V, 0.35, B)
        assert np.allclose(a, b, rtol=0, atol=1e-13) == same


def test_pin_partition_merge_matches_full_softmax():
    rng = _rng(12)
    D = 8
    for n in (1, 15, 16, 17, 100, 513):
        q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
        full = P.attention(q, K, V, 0.5)
        for ps in (1, 16, 64, 512, 4096):
            np.testing.assert_allclose(P.partitioned_attention(q, K, V, 0.5, ps), full,
                                       rtol=0, atol=1e-13)
    # scores shifted far apart: the rescaling by e^(m_p - M) matters
    K = rng.standard_normal((64, D))
    q = rng.standard_normal(D) * 20
    V = rng.standard_normal((64, D))
    np.testing.assert_allclose(P.partitioned_attention(q, K, V, 1.0, 16), P.attention(q, K, V, 1.0),
                               rtol=0, atol=1e-12)


def test_pin_empty_context_and_masked_slots():
    """n = 0 gives zeros; NaN in slots past the context never reaches the
    result (the oracle only reads tokens < n)."""
    wl = make_workload(0)
    assert np.isnan(wl.key_cache.astype(np.float64)).any()       # the generator poisoned tails
    out = P.paged_decode(wl.q, wl.key_cache, wl.value_cache, wl.block_tables, wl.context_lens,
                         wl.block_size, wl.scale, wl.dtype)
    assert np.isfinite(out).all()
    z = P.attention(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.array_equal(z, np.zeros(4))


def test_pin_dtype_decoding():
    """bf16 words decode to the float32 with the same top 16 bits; fp16 and
    fp32 decode to their IEEE values; rounding back is exact."""
    words = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F80, 0x3E20], dtype=np.uint16)
    vals = P.to_f64(words, "bf16")
    assert vals.tolist()[:4] == [1.0, -1.0, 3.140625, 0.0]
    assert vals[4] == float("inf") and vals[5] == 0.15625
    h = np.array([1.0, -2.5, 65504.0, 6e-8], dtype=np.float16)
    assert np.array_equal(P.to_f64(h, "f16"), h.astype(np.float64))
    x = np.array([1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9, -3.0 - 2 ** -8])
    assert P.round_to_dtype(x, "bf16").tolist() == [1.0, 1.0 + 2 ** -7, -3.0]


def test_pin_kv_bytes_page2():
    g = _golden("p2_kv_bytes.json")
    assert P.kv_cache_bytes(g["seq_len"], g["num_layers"], g["num_heads"], g["head_dim"],
                            g["dtype_size"]) == g["bytes"]


def test_pin_gqa_group_one_is_mha():
    """G = 1 maps head h to kv head h; G > 1 maps consecutive groups."""
    assert [P.kv_head_of(h, 8, 8) for h in range(8)] == list(range(8))
    assert [P.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


@pytest.mark.parametrize("idx", [0])
def test_workload_tiny_shape(idx):
    """The tiny fp32 workload has the stated shape: 4 sequences of 17, 50, 128
    and 200 tokens in disjoint slices of a 64-block pool."""
    wl = make_workload(idx)
    assert wl.context_lens.tolist() == [17, 50, 128, 200]
    used = [P.num_required_blocks(int(n), 16) for n in wl.context_lens]
    assert used == [2, 4, 8, 13]
    ids = np.concatenate([wl.block_tables[s, :used[s]] for s in range(4)])
    assert len(set(ids.tolist())) == 27 and ids.min() >= 0 and ids.max() < 64
    assert wl.key_cache.shape == (64, 8, 16, 64)


def test_workload_f16_rounding_is_numpys_cast():
    """The generators' float32 -> fp16 rounding (integer ufuncs, so chunks
    convert in parallel) gives numpy's own cast's words for every non-NaN
    float32: random bit patterns, the subnormal and overflow boundaries, and
    every float32 around the smallest normal."""
    import warnings

    import workloads as W
    rng = _rng(44)
    pats = [rng.integers(0, 2**32, 1 << 20, dtype=np.uint64).astype(np.uint32),
            np.arange(0x33000000, 0x39000000, 97, dtype=np.uint32),
            np.arange(0x477F0000, 0x7F800001, 4099, dtype=np.uint32)]
    for p in pats:
        for x in (p.view(np.float32), -p.view(np.float32)):
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                want = x.astype(np.float16).view(np.uint16)
            got = W._f32_to_f16_bits(x)
            keep = ~np.isnan(x)
            assert np.array_equal(got[keep], want[keep])
            assert ((got[~keep] & 0x7FFF) == 0x7E00).all()


def test_workload_reproducible_and_prefix_shared():
    a = build("t", "bf16", [70, 130], 4, 2, 16, 16, seed=3, shared_prefix_tokens=32)
    b = build("t", "bf16", [70, 130], 4, 2, 16, 16, seed=3, shared_prefix_tokens=32)
    assert np.array_equal(a.key_cache, b.key_cache) and np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.block_tables[0, :2], a.block_tables[1, :2])


# --------------------------------------------------------------------------
# Whole-block copies (swap out / in, copy on write)
# --------------------------------------------------------------------------

def test_pin_copy_blocks_swap_round_trip_keeps_attention():
    """Swapping a request's blocks out to a host pool and back in to other
    device blocks (P3 §3, §5), with its table rewritten to the new ids, leaves
    the pool contents it reads -- and so its attention output -- bit for bit
    unchanged; blocks named by no pair are untouched; out-of-range pairs are
    skipped."""
    rng = _rng(31)
    NB, Hkv, B, D, n = 12, 2, 4, 8, 13
    kc = rng.standard_normal((NB, Hkv, B, D)).astype(np.float32)
    vc = rng.standard_normal((NB, Hkv, B, D)).astype(np.float32)
    table = [7, 2, 9, 4]
    q = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    before = P.paged_decode(q, kc, vc, np.array([table], np.int32), np.array([n], np.int32), B,
                            0.3, "f32")
    host_k = np.full((6, Hkv, B, D), -7.0, np.float32)
    host_v = np.full((6, Hkv, B, D), -7.0, np.float32)
    out_pairs = [(b, i) for i, b in enumerate(table)] + [(99, 0), (0, 99)]
    P.copy_blocks(host_k, kc, out_pairs)
    P.copy_blocks(host_v, vc, out_pairs)
    for i, b in enumerate(table):
        assert host_k[i].tobytes() == kc[b].tobytes() and host_v[i].tobytes() == vc[b].tobytes()
    assert (host_k[4:] == -7.0).all() and (host_v[4:] == -7.0).all()
    # the request's device blocks are reused by someone else meanwhile
    kc2, vc2 = kc.copy(), vc.copy()
    for b in table:
        kc2[b] = np.nan
        vc2[b] = np.nan
    new_table = [0, 11, 5, 3]
    in_pairs = [(i, b) for i, b in enumerate(new_table)]
    untouched = [b for b in range(NB) if b not in new_table]
    snap = kc2[untouched].tobytes()
    P.copy_blocks(kc2, host_k, in_pairs)
    P.copy_blocks(vc2, host_v, in_pairs)
    assert kc2[untouched].tobytes() == snap
    after = P.paged_decode(q, kc2, vc2, np.array([new_table], np.int32), np.array([n], np.int32),
                           B, 0.3, "f32")
    assert after.tobytes() == before.tobytes()


# --------------------------------------------------------------------------
# 8-bit (E4M3) KV storage
# --------------------------------------------------------------------------

def test_pin_e4m3_decode_library_and_spec_values():
    """All 256 codes against torch's float8_e4m3fn (library routine) and the
    format's landmark values (1.0, largest finite 448, smallest normal 2^-6,
    smallest subnormal 2^-9, negative zero, NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    got = P.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], lib[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(lib[~nan]))
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6
    assert got[0x01] == 2.0 ** -9 and got[0x80] == 0.0 and np.signbit(got[0x80])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0xFE] == -448.0


def test_pin_e4m3_encode_nearest_ties_even_saturating():
    """Encoding is the nearest code by brute force over every finite code,
    ties to the even code; it agrees with torch in range (random values and
    every midpoint between neighbouring codes), saturates at +-448 beyond
    (torch gives NaN there: the reading here saturates), and round-trips
    every finite code."""
    vals = P.e4m3_decode(np.arange(0x7F, dtype=np.uint8))          # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    rng = _rng(7)
    x = np.concatenate([rng.standard_normal(3000) * 40, mids, -mids, vals, -vals,
                        rng.uniform(-460, 460, 2000)]).astype(np.float32).astype(np.float64)
    enc = P.e4m3_encode(x)
    lib = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc, lib)
    finite = np.arange(256)[(np.arange(256) & 0x7F) != 0x7F].astype(np.uint8)
    fv = P.e4m3_decode(finite)
    for xv, c in zip(x[:600], enc[:600]):
        d = np.abs(fv - xv)
        best = finite[d == d.min()]
        if len(best) > 1:                                           # a tie (or +-0)
            best = [b for b in best if (b & 1) == 0 and np.signbit(P.e4m3_decode(b)) == np.signbit(xv)] or best
        assert c in best
    assert P.e4m3_encode(np.array([500.0, 1e6, -1e6, 464.0, np.nan])).tolist() == [0x7E, 0x7E, 0xFE, 0x7E, 0x7F]
    assert np.array_equal(P.e4m3_encode(P.e4m3_decode(finite)), finite)


def test_pin_fp8_decode_is_attention_on_dequantized_values():
    """Decode over E4M3 pools equals the library attention routine (float64
    SDPA) on the gathered context's values code * scale."""
    rng = _rng(8)
    NB, H, Hkv, B, D = 10, 4, 2, 16, 64
    kc = P.e4m3_encode(rng.standard_normal((NB, Hkv, B, D)) * 3)
    vc = P.e4m3_encode(rng.standard_normal((NB, Hkv, B, D)) * 3)
    q = rng.standard_normal((1, H, D)).astype(np.float16)
    table = np.array([[6, 2, 9, 0]], np.int32)
    n = 57
    got = P.paged_decode_fp8(q, kc, vc, table, np.array([n], np.int32), B, 0.125, "f16", 0.75, 1.5)
    rows = [table[0][t // B] for t in range(n)]
    offs = [t % B for t in range(n)]
    Kc = torch.tensor(P.e4m3_decode(kc[rows, :, offs, :]) * 0.75)     # [n][Hkv][D]
    Vc = torch.tensor(P.e4m3_decode(vc[rows, :, offs, :]) * 1.5)
    G = H // Hkv
    qt = torch.tensor(P.to_f64(q, "f16"))[0]                            # [H][D]
    for h in range(H):
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[h][None, None], Kc[:, h // G][None], Vc[:, h // G][None], scale=0.125)[0, 0].numpy()
        assert np.abs(got[0, h] - ref).max() < 1e-12


def test_pin_fp8_cache_write_quantises_with_pool_scale():
    """The fp8 cache write stores encode(float32(x) / scale) for each new row
    in its slot and leaves other slots untouched; decode(code) * scale is
    within half a code spacing of x."""
    rng = _rng(9)
    NB, Hkv, B, D = 6, 2, 4, 16
    kc = np.full((NB, Hkv, B, D), 0x55, np.uint8)
    vc = kc.copy()
    key = rng.standard_normal((3, Hkv, D)).astype(np.float16)
    val = rng.standard_normal((3, Hkv, D)).astype(np.float16)
    slots = np.array([5, 22, -1], np.int64)
    P.cache_write_fp8(kc, vc, key, val, slots, B, "f16", 0.01, 0.02)
    for i, slot in enumerate(slots[:2]):
        b, o = slot // B, slot % B
        xk = key[i].astype(np.float64)
        back = P.e4m3_decode(kc[b, :, o, :]) * np.float64(np.float32(0.01))
        spacing = np.maximum(np.exp2(np.floor(np.log2(np.abs(xk / 0.01) + 1e-30)) - 3), 2.0 ** -9)
        assert (np.abs(back - xk) <= 0.5 * spacing * 0.01 * (1 + 1e-6)).all()
    touched = np.zeros((NB, B), bool)
    touched[5 // B, 5 % B] = touched[22 // B, 22 % B] = True
    assert (kc.transpose(0, 2, 1, 3)[~touched] == 0x55).all()


def test_pin_fp8_quantiser_divides_in_float32():
    """Reading F1: the stored code is the one nearest float32(x) / float32(s),
    the quotient rounded to float32 (the kernel's precision).  On inputs
    where the exact quotient (float64) lands on another code, the oracle
    must give the float32 quotient's code (brute force over torch's E4M3
    table), for both signs and for inputs of every source type."""
    for src in ("f32", "f16", "bf16"):
        for scale in (FP8C.K_SCALE, FP8C.V_SCALE):
            cases = FP8C.divergent_inputs(src, scale)
            assert len(cases) >= 8, f"only {len(cases)} divergent inputs for {src} at {scale}"
            xs = np.array([x for x, _, _ in cases] + [-x for x, _, _ in cases], np.float32)
            want32 = [c32 for _, c32, _ in cases] + [c32 | 0x80 for _, c32, _ in cases]
            want64 = [c64 for _, _, c64 in cases] + [c64 | 0x80 for _, _, c64 in cases]
            got = P.quantize_e4m3(xs, scale)
            assert got.tolist() == want32, f"{src} at scale {scale}"
            assert all(g != w for g, w in zip(got.tolist(), want64))


# --------------------------------------------------------------------------
# Paged prefill
# --------------------------------------------------------------------------

def _prefill_case(seed, ctx, qlens, H, Hkv, D, B, dtype="f32"):
    rng = _rng(seed)
    S = len(ctx)
    nb = [P.num_required_blocks(c, B) for c in ctx]
    NB = sum(nb) + 3
    perm = rng.permutation(NB)
    MB = max(nb)
    tables = np.full((S, MB), -1, np.int32)
    pos = 0
    for s in range(S):
        tables[s, :nb[s]] = perm[pos:pos + nb[s]]
        pos += nb[s]
    kc = rng.standard_normal((NB, Hkv, B, D)).astype(np.float32)
    vc = rng.standard_normal((NB, Hkv, B, D)).astype(np.float32)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), H, D)).astype(np.float32)
    return kc, vc, tables, np.array(ctx, np.int32), qs, q


def _contiguous(cache, table, n, B):
    return np.stack([cache[table[t // B], :, t % B, :] for t in range(n)])   # [n][Hkv][D]


def test_pin_prefill_fresh_prompts_are_causal_sdpa():
    """A whole prompt as queries (qlen = ctx) is causal attention over the
    contiguous sequence: the library routine with is_causal (float64), with
    kv heads repeated for grouped queries."""
    B, H, Hkv, D = 4, 4, 2, 8
    ctx = [9, 1, 13]
    kc, vc, tables, cl, qs, q = _prefill_case(40, ctx, ctx, H, Hkv, D, B)
    got = P.paged_prefill(q, kc, vc, tables, cl, qs, B, 0.4, "f32")
    G = H // Hkv
    for s, n in enumerate(ctx):
        K = torch.tensor(_contiguous(kc, tables[s], n, B).astype(np.float64)).repeat_interleave(G, 1)
        V = torch.tensor(_contiguous(vc, tables[s], n, B).astype(np.float64)).repeat_interleave(G, 1)
        Q = torch.tensor(q[qs[s]:qs[s + 1]].astype(np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q.transpose(0, 1), K.transpose(0, 1), V.transpose(0, 1), is_causal=True,
            scale=0.4).transpose(0, 1).numpy()
        assert np.abs(got[qs[s]:qs[s + 1]] - ref).max() < 1e-12


def test_pin_prefill_suffix_after_cached_prefix():
    """Queries for only the last qlen tokens (the prefix is already cached, as
    with a shared prefix): row j attends to tokens 0 .. ctx - qlen + j, the
    library routine with that explicit mask."""
    B, H, Hkv, D = 8, 2, 2, 16
    ctx, qlens = [40, 17, 64], [5, 17, 1]
    kc, vc, tables, cl, qs, q = _prefill_case(41, ctx, qlens, H, Hkv, D, B)
    got = P.paged_prefill(q, kc, vc, tables, cl, qs, B, 0.25, "f32")
    for s, (n, L) in enumerate(zip(ctx, qlens)):
        K = torch.tensor(_contiguous(kc, tables[s], n, B).astype(np.float64)).transpose(0, 1)
        V = torch.tensor(_contiguous(vc, tables[s], n, B).astype(np.float64)).transpose(0, 1)
        Q = torch.tensor(q[qs[s]:qs[s + 1]].astype(np.float64)).transpose(0, 1)
        mask = torch.tensor([[t <= n - L + j for t in range(n)] for j in range(L)])
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                               scale=0.25).transpose(0, 1).numpy()
        assert np.abs(got[qs[s]:qs[s + 1]] - ref).max() < 1e-12


def test_pin_prefill_last_row_is_decode():
    """The last query row of a sequence is the decode output for that
    sequence (same context)."""
    B, H, Hkv, D = 4, 4, 4, 8
    ctx, qlens = [11, 30], [3, 30]
    kc, vc, tables, cl, qs, q = _prefill_case(42, ctx, qlens, H, Hkv, D, B)
    got = P.paged_prefill(q, kc, vc, tables, cl, qs, B, 0.3, "f32")
    last = q[qs[1:] - 1]                                        # [S][H][D]
    dec = P.paged_decode(last, kc, vc, tables, cl, B, 0.3, "f32")
    assert np.array_equal(got[qs[1:] - 1], dec)


def _fp8_prefill_case(seed, ctx, qlens, H, Hkv, D, B):
    from workloads import e4m3_codes, normal_array
    rng = np.random.default_rng(seed)
    nblk = [-(-c // B) for c in ctx]
    NB = sum(nblk) + 3
    ids = rng.permutation(NB)
    tables = np.full((len(ctx), max(nblk)), -1, np.int32)
    k = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = ids[k:k + n]
        k += n
    kc = e4m3_codes(seed, 1, (NB, Hkv, B, D))
    vc = e4m3_codes(seed, 2, (NB, Hkv, B, D))
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = normal_array(seed, 3, (int(qs[-1]), H, D), "f16")
    return kc, vc, tables, np.array(ctx, np.int32), qs, q


def test_pin_prefill_fp8_is_prefill_over_the_decoded_pools():
    """Prefill over E4M3 pools equals prefill over float32 pools holding
    decode(code) * scale (exact: E4M3 values times a power of two are
    float32 values) with the fp16 queries widened exactly: the codes are
    gathered through the table at the causal positions and scaled per pool."""
    B, H, Hkv, D = 4, 4, 2, 8
    ctx, qlens = [11, 30, 5], [3, 30, 5]
    kc, vc, tables, cl, qs, q = _fp8_prefill_case(61, ctx, qlens, H, Hkv, D, B)
    ks, vs = 0.5, 0.25
    got = P.paged_prefill_fp8(q, kc, vc, tables, cl, qs, B, 0.3, "f16", ks, vs, Hkv)
    kf = (P.e4m3_decode(kc) * ks).astype(np.float32)
    vf = (P.e4m3_decode(vc) * vs).astype(np.float32)
    assert np.array_equal(kf.astype(np.float64), P.e4m3_decode(kc) * ks)
    q32 = P.to_f64(q, "f16").astype(np.float32)
    ref = P.paged_prefill(q32, kf, vf, tables, cl, qs, B, 0.3, "f32", Hkv)
    assert np.array_equal(got, ref)
    # the K scale acts as a factor of the score scale
    got2 = P.paged_prefill_fp8(q, kc, vc, tables, cl, qs, B, 0.15, "f16", 2 * ks, vs, Hkv)
    assert np.allclose(got2, got, rtol=0, atol=1e-12)


def test_pin_prefill_fp8_last_row_is_fp8_decode():
    B, H, Hkv, D = 4, 4, 4, 8
    ctx, qlens = [9, 22], [4, 22]
    kc, vc, tables, cl, qs, q = _fp8_prefill_case(62, ctx, qlens, H, Hkv, D, B)
    got = P.paged_prefill_fp8(q, kc, vc, tables, cl, qs, B, 0.3, "f16", 0.5, 0.5)
    last = q[qs[1:] - 1]
    dec = P.paged_decode_fp8(last, kc, vc, tables, cl, B, 0.3, "f16", 0.5, 0.5)
    assert np.array_equal(got[qs[1:] - 1], dec)
