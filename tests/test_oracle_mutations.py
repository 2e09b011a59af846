"""Plant plausible mistakes in the oracle (on the CPU) and check that the pin
suite catches every one of them.  Each mutant replaces one oracle function;
the test passes when at least one pin fails (an assertion or an exception)."""
import math

import numpy as np
import pytest

import oracle.paged as P
import tests.test_oracle_pins as pins

_orig = {name: getattr(P, name) for name in dir(P) if callable(getattr(P, name))}

PINS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_pin_")]


def _floor_blocks(n, b):
    return n // b


def _swapped_location(table_row, t, b):
    logical, offset = t % b, t // b
    if logical >= len(table_row) or table_row[logical] < 0:
        return None
    return int(table_row[logical]), offset


def _off_by_one_location(table_row, t, b):
    return _orig["physical_location"](table_row, t + 1, b) if t + 1 < len(table_row) * b else \
        _orig["physical_location"](table_row, t, b)


def _no_scale(q, K, V, scale):
    return _orig["attention"](q, K, V, 1.0)


def _wrong_sign(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[-1])
    s = scale * (K @ q)
    w = np.exp(s.max() - s)
    return (w @ V) / w.sum()


def _mean_normaliser(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[-1])
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w @ V) / len(w)


def _keys_as_values(q, K, V, scale):
    return _orig["attention"](q, K, K if K.shape == V.shape else V, scale)


def _blockwise(q, K, V, scale):
    return _orig["blockwise_softmax_sum"](q, K, V, scale, 16)


def _mod_heads(h, H, Hkv):
    return h % Hkv


def _merge_without_rescale(states):
    live = [(m, l, o) for m, l, o in states if m != float("-inf")]
    if not live:
        return np.zeros(states[0][2].shape[-1])
    return sum(o for _, _, o in live) / sum(l for _, l, _ in live)


def _cache_write_key_twice(kc, vc, key, value, slots, b):
    return _orig["cache_write"](kc, vc, key, key, slots, b)


def _cache_write_no_bounds(kc, vc, key, value, slots, b):
    nb = kc.shape[0]
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        slot = int(slot) % (nb * b)
        kc[slot // b, :, slot % b, :] = key[i]
        vc[slot // b, :, slot % b, :] = value[i]


def _slots_last_plus_one(block_tables, block_size, num_blocks, context_lens=None, seq_ids=None,
                         positions=None):
    if positions is None and context_lens is not None:
        context_lens = np.asarray(context_lens) + 1
    return _orig["compute_slots"](block_tables, block_size, num_blocks, context_lens, seq_ids, positions)


def _bf16_wrong_shift(raw, dtype):
    if dtype == "bf16":
        w = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return w.view(np.float32).astype(np.float64)
    return _orig["to_f64"](raw, dtype)


def _kv_bytes_no_two(seq_len, layers, heads, hd, e):
    return seq_len * layers * heads * hd * e


def _copy_reversed(dst_pool, src_pool, pairs):
    return _orig["copy_blocks"](dst_pool, src_pool, [(d, s) for s, d in pairs])


def _copy_no_bounds(dst_pool, src_pool, pairs):
    for s, d in pairs:
        dst_pool[int(d) % dst_pool.shape[0]] = src_pool[int(s) % src_pool.shape[0]]


def _e4m3_bias8(codes):
    return _orig["e4m3_decode"](codes) / 2.0


def _e4m3_no_subnormals(codes):
    c = np.asarray(codes, dtype=np.uint8)
    v = _orig["e4m3_decode"](c)
    return np.where(((c >> 3) & 0xF) == 0, 0.0, v)


def _e4m3_truncate(x):
    v = np.asarray(x, dtype=np.float64)
    table = _orig["e4m3_decode"](np.arange(0x7F, dtype=np.uint8))
    out = np.empty(v.shape, np.uint8)
    for i, xv in enumerate(v.reshape(-1)):
        a = min(abs(xv), 448.0)
        j = int(np.searchsorted(table, a, side="right")) - 1
        out.reshape(-1)[i] = j | (0x80 if xv < 0 else 0)
    return out


def _e4m3_ties_up(x):
    v = np.asarray(x, dtype=np.float64)
    table = _orig["e4m3_decode"](np.arange(0x7F, dtype=np.uint8))
    out = np.empty(v.shape, np.uint8)
    for i, xv in enumerate(v.reshape(-1)):
        a = min(abs(xv), 448.0)
        j = int(np.argmin(np.abs(table - a) - 1e-12 * np.arange(len(table))))
        out.reshape(-1)[i] = j | (0x80 if xv < 0 else 0)
    return out


def _quantize_times_scale(x_f32, scale):
    return _orig["e4m3_encode"]((np.asarray(x_f32, np.float32) * np.float32(scale)).astype(np.float64))


def _fp8_decode_no_v_scale(q, kc, vc, bt, cl, b, scale, qd, ks, vs, hkv=None, pairs=None):
    return _orig["paged_decode_fp8"](q, kc, vc, bt, cl, b, scale, qd, ks, 1.0, hkv, pairs)


def _prefill_top_left(q, kc, vc, bt, cl, qs, b, scale, dtype, hkv=None, rows=None):
    cl2 = np.array([int(qs[s + 1]) - int(qs[s]) for s in range(len(cl))], np.int32)
    return _orig["paged_prefill"](q, kc, vc, bt, cl2, qs, b, scale, dtype, hkv, rows)


def _prefill_not_causal(q, kc, vc, bt, cl, qs, b, scale, dtype, hkv=None, rows=None):
    T = q.shape[0]
    qs2 = np.arange(T + 1) * 0
    out = np.empty((T,) + q.shape[1:])
    for s in range(len(cl)):
        for i in range(int(qs[s]), int(qs[s + 1])):
            out[i] = _orig["paged_decode"](q[i:i + 1], kc, vc, bt[s:s + 1], cl[s:s + 1], b, scale,
                                           dtype, hkv)[0]
    return out


def _prefill_pos_plus_one(q, kc, vc, bt, cl, qs, b, scale, dtype, hkv=None, rows=None):
    T, H, D = q.shape
    out = np.full((T, H, D), np.nan)
    Hk = kc.shape[1] if hkv is None else hkv
    for s in range(len(cl)):
        L = int(qs[s + 1]) - int(qs[s])
        for j in range(L):
            n = min(int(cl[s]) - L + j + 2, int(cl[s]))
            for h in range(H):
                out[int(qs[s]) + j, h] = P.decode_one(P.to_f64(q[int(qs[s]) + j, h], dtype), kc, vc,
                                                      bt[s], n, P.kv_head_of(h, H, Hk), b, scale, dtype)
    return out


def _quantize_exact_division(x_f32, scale):
    q = np.asarray(x_f32, dtype=np.float32).astype(np.float64) / float(np.float32(scale))
    return _orig["e4m3_encode"](q)


MUTANTS = {
    "paged_prefill": [_prefill_top_left, _prefill_not_causal, _prefill_pos_plus_one],
    "e4m3_decode": [_e4m3_bias8, _e4m3_no_subnormals],
    "e4m3_encode": [_e4m3_truncate, _e4m3_ties_up],
    "quantize_e4m3": [_quantize_times_scale, _quantize_exact_division],
    "paged_decode_fp8": [_fp8_decode_no_v_scale],
    "copy_blocks": [_copy_reversed, _copy_no_bounds],
    "num_required_blocks": [_floor_blocks],
    "physical_location": [_swapped_location, _off_by_one_location],
    "attention": [_no_scale, _wrong_sign, _mean_normaliser, _keys_as_values, _blockwise],
    "kv_head_of": [_mod_heads],
    "merge_partitions": [_merge_without_rescale],
    "cache_write": [_cache_write_key_twice, _cache_write_no_bounds],
    "compute_slots": [_slots_last_plus_one],
    "to_f64": [_bf16_wrong_shift],
    "kv_cache_bytes": [_kv_bytes_no_two],
}

CASES = [(name, fn) for name, fns in MUTANTS.items() for fn in fns]


@pytest.mark.parametrize("name,mutant", CASES, ids=[f"{n}:{f.__name__}" for n, f in CASES])
def test_pins_catch_mutant(name, mutant, monkeypatch):
    monkeypatch.setattr(P, name, mutant)
    failures = 0
    for pin in PINS:
        try:
            pin()
        except (Exception, pytest.fail.Exception):   # an assertion or a crash both count
            failures += 1
    assert failures > 0, f"no pin detects the mutant {mutant.__name__} of {name}"


def test_unmutated_oracle_passes_every_pin():
    for pin in PINS:
        pin()
    assert math.isfinite(len(PINS)) and len(PINS) >= 15
