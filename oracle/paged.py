"""Plain float64 reference for paged decode, cache write and slot resolution.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may use it and for
the source keys P1, P2, P3).  Slow and obvious on purpose: per-sequence,
per-head numpy in float64, no blocking or fusion beyond what the definitions
state.

Storage conventions (the pages fix none; these are the plain readings):
pools are ``[num_blocks][num_kv_heads][block_size][head_dim]`` of raw storage
words (float32, float16, or bfloat16 as uint16); ``q`` and the output are
``[num_seqs][num_heads][head_dim]``; tables are int32 ``[num_seqs][max_blocks]``.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


# ---------------------------------------------------------------------------
# Slot arithmetic -- P3 §3 (the Rust block-table helper: logical block =
# token index / block size, offset = token index % block size, physical id =
# table[logical]; blocks needed = ceil(tokens / block size)).
# ---------------------------------------------------------------------------

def num_required_blocks(num_tokens: int, block_size: int) -> int:
    """Blocks needed to hold ``num_tokens`` tokens (P3 §3, rounding up)."""
    return (num_tokens + block_size - 1) // block_size


def physical_location(table_row, token_idx: int, block_size: int):
    """(physical block, offset) of token ``token_idx`` or None past the table
    (P3 §3: the lookup returns nothing when the logical block has no entry)."""
    logical = token_idx // block_size
    offset = token_idx % block_size
    if logical >= len(table_row):
        return None
    phys = int(table_row[logical])
    if phys < 0:
        return None
    return phys, offset


def slot_of(table_row, token_idx: int, block_size: int) -> int:
    """Flat slot index phys * B + offset, or -1 when the token has no block."""
    loc = physical_location(table_row, token_idx, block_size)
    if loc is None:
        return -1
    return loc[0] * block_size + loc[1]


def compute_slots(block_tables, block_size: int, num_blocks: int, context_lens=None,
                  seq_ids=None, positions=None) -> np.ndarray:
    """Slots of a batch of tokens.

    Token i belongs to sequence ``seq_ids[i]`` (or i when absent) and sits at
    ``positions[i]`` (or, when absent, at the newest position of that sequence,
    ``context_lens[seq] - 1``: P2 §2.1 appends the new token's K/V before
    attending).  A token whose position is negative, whose logical block is past
    the table, or whose table entry is outside ``[0, num_blocks)`` gets -1.
    """
    tables = np.asarray(block_tables)
    n = len(positions) if positions is not None else (
        len(seq_ids) if seq_ids is not None else tables.shape[0])
    out = np.full(n, -1, dtype=np.int64)
    for i in range(n):
        s = int(seq_ids[i]) if seq_ids is not None else i
        if s < 0 or s >= tables.shape[0]:
            continue
        pos = int(positions[i]) if positions is not None else int(context_lens[s]) - 1
        if pos < 0:
            continue
        loc = physical_location(tables[s], pos, block_size)
        if loc is None or loc[0] >= num_blocks:
            continue
        out[i] = loc[0] * block_size + loc[1]
    return out


# ---------------------------------------------------------------------------
# Whole-block copies -- P3 §4 (a beam fork shares block references; a writer
# into a shared block needs a private copy) and P3 §3, §5 (blocks of a
# preempted request are swapped out to CPU memory and back in).
# ---------------------------------------------------------------------------

def copy_blocks(dst_pool, src_pool, pairs) -> None:
    """``dst_pool[d] = src_pool[s]`` bit for bit for each (s, d) pair whose ids
    lie inside their pools; other pairs are skipped.  Pools are arrays whose
    first axis is the physical block id."""
    for s_id, d_id in pairs:
        s_id, d_id = int(s_id), int(d_id)
        if 0 <= s_id < src_pool.shape[0] and 0 <= d_id < dst_pool.shape[0]:
            dst_pool[d_id] = src_pool[s_id]


# ---------------------------------------------------------------------------
# Storage decoding
# ---------------------------------------------------------------------------

def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of raw storage words ("f64": already values)."""
    if dtype == "f64":
        return np.asarray(raw, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(raw, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        w = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return w.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` (nearest, ties to even) and return
    them as float64 again.  bf16 rounds the float64 significand to 8 bits
    directly (normal range), so there is no double rounding through float32."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        m, e = np.frexp(x)                  # x = m * 2**e, 0.5 <= |m| < 1
        return np.ldexp(np.rint(m * 256.0) / 256.0, e)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Cache write -- P2 §2.1 step 3 (the new token's K and V join the cache) at
# the slot P3 §3 assigns.  A raw-bit copy; the pools are modified in place.
# ---------------------------------------------------------------------------

def cache_write(key_cache: np.ndarray, value_cache: np.ndarray, key: np.ndarray,
                value: np.ndarray, slot_mapping, block_size: int) -> None:
    """``cache[slot // B][h][slot % B][:] = key[i][h][:]`` for every token i
    whose slot lies in ``[0, num_blocks * B)``; other slots are skipped."""
    nb = key_cache.shape[0]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        slot = int(slot)
        if slot < 0 or slot >= nb * block_size:
            continue
        blk, off = slot // block_size, slot % block_size
        key_cache[blk, :, off, :] = key[i]
        value_cache[blk, :, off, :] = value[i]


# ---------------------------------------------------------------------------
# Gather and attention
# ---------------------------------------------------------------------------

def gather_context(cache: np.ndarray, table_row, n: int, kv_head: int,
                   block_size: int) -> np.ndarray:
    """Rows of tokens 0..n-1 of one kv head as a contiguous ``[n][D]`` array
    (same element type as ``cache``): look each token up through the table
    (P3 §2, §3) and concatenate, as the block-joining helper of P1 §7 does."""
    D = cache.shape[-1]
    out = np.empty((n, D), dtype=cache.dtype)
    for t in range(n):
        loc = physical_location(table_row, t, block_size)
        if loc is None:
            raise ValueError(f"token {t} has no block in the table")
        phys, off = loc
        if not (0 <= phys < cache.shape[0]):
            raise ValueError(f"block id {phys} outside the pool")
        out[t] = cache[phys, kv_head, off]
    return out


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for one query row (P1 §1, first formula;
    P2 §2.1 steps 4-5).  An empty context gives zeros (the pages are silent)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[-1], dtype=np.float64)
    s = scale * (K @ q)
    m = s.max()
    w = np.exp(s - m)
    return (w @ V) / w.sum()


def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """Grouped-query mapping: consecutive groups of H / Hkv query heads share
    one kv head (a convention: the pages do not treat grouped queries)."""
    return h // (num_heads // num_kv_heads)


def decode_one(q_row64: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray, table_row,
               n: int, kv_head: int, block_size: int, scale: float,
               dtype: str | None = None) -> np.ndarray:
    """Decode output of one (sequence, head): gather, widen to float64 (when
    ``dtype`` names the pools' storage type), then attend."""
    K = gather_context(key_cache, table_row, n, kv_head, block_size)
    V = gather_context(value_cache, table_row, n, kv_head, block_size)
    if dtype is not None:
        K, V = to_f64(K, dtype), to_f64(V, dtype)
    return attention(q_row64, K, V, scale)


def paged_decode(q, key_cache, value_cache, block_tables, context_lens, block_size: int,
                 scale: float, dtype: str, num_kv_heads: int | None = None,
                 pairs=None) -> np.ndarray:
    """Float64 decode output ``[S][H][D]`` (or only the listed (s, h) pairs,
    others left NaN)."""
    q64 = to_f64(q, dtype)
    S, H, D = q64.shape
    Hkv = key_cache.shape[1] if num_kv_heads is None else num_kv_heads
    if H % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    out = np.full((S, H, D), np.nan)
    todo = pairs if pairs is not None else [(s, h) for s in range(S) for h in range(H)]
    for s, h in todo:
        n = int(context_lens[s])
        out[s, h] = decode_one(q64[s, h], key_cache, value_cache, block_tables[s], n,
                               kv_head_of(h, H, Hkv), block_size, scale, dtype)
    return out


# ---------------------------------------------------------------------------
# Paged prefill.  The pages give the per-token step (P2 §2.1: the token's K/V
# join the cache, then its query attends over every cached K/V) and say that
# prompts sharing a cached prefix skip that prefix's prefill work (P3 §3,
# prefix sharing saves 50-80% of prefill).  Reading: the last ``qlen`` tokens
# of a sequence's context are queries; query row j sits at position
# p = ctx - qlen + j and attends causally to tokens 0..p, gathered through
# the block table -- the decode formula at every position.
# ---------------------------------------------------------------------------

def paged_prefill(q, key_cache, value_cache, block_tables, context_lens, query_start,
                  block_size: int, scale: float, dtype: str,
                  num_kv_heads: int | None = None, rows=None) -> np.ndarray:
    """Float64 prefill output ``[T][H][D]`` for query rows ``q [T][H][D]``;
    sequence s owns rows query_start[s] .. query_start[s+1]-1.  ``rows``
    (optional) lists (row, head) pairs to compute; others stay NaN."""
    q64 = to_f64(q, dtype)
    T, H, D = q64.shape
    Hkv = key_cache.shape[1] if num_kv_heads is None else num_kv_heads
    if H % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    seq_of = np.full(T, -1, dtype=np.int64)
    for s in range(len(context_lens)):
        seq_of[int(query_start[s]):int(query_start[s + 1])] = s
    out = np.full((T, H, D), np.nan)
    todo = rows if rows is not None else [(i, h) for i in range(T) for h in range(H)]
    for i, h in todo:
        s = int(seq_of[i])
        qlen = int(query_start[s + 1]) - int(query_start[s])
        pos = int(context_lens[s]) - qlen + (i - int(query_start[s]))
        out[i, h] = decode_one(q64[i, h], key_cache, value_cache, block_tables[s], pos + 1,
                               kv_head_of(h, H, Hkv), block_size, scale, dtype)
    return out

# ---------------------------------------------------------------------------
# Split-context partitions and their log-sum-exp merge.  Not on the pages:
# the plain way to evaluate the full softmax of P1 §1 over pieces of the
# context.  (P1 §1's second formula, a sum of per-block softmaxes, is a
# different quantity once there is more than one block; see
# ``blockwise_softmax_sum``.)
# ---------------------------------------------------------------------------

def partition_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                    start: int, stop: int):
    """(m, l, o) of tokens [start, stop): m = max score, l = sum exp(s - m),
    o = sum exp(s - m) v (unnormalised).  Empty range: (-inf, 0, 0)."""
    if stop <= start:
        return NEG_INF, 0.0, np.zeros(V.shape[-1])
    s = scale * (K[start:stop] @ q)
    m = s.max()
    w = np.exp(s - m)
    return float(m), float(w.sum()), w @ V[start:stop]


def merge_partitions(states) -> np.ndarray:
    """Combine partition states: M = max m_p; out = sum e^(m_p - M) o_p /
    sum e^(m_p - M) l_p.  All-empty gives zeros."""
    ms = [m for m, _, _ in states]
    D = states[0][2].shape[-1]
    if all(m == NEG_INF for m in ms):
        return np.zeros(D)
    M = max(ms)
    num = np.zeros(D)
    den = 0.0
    for m, l, o in states:
        if m == NEG_INF:
            continue
        w = math.exp(m - M)
        num = num + w * o
        den += w * l
    return num / den


def partitioned_attention(q, K, V, scale: float, partition_size: int) -> np.ndarray:
    n = K.shape[0]
    states = [partition_state(q, K, V, scale, p, min(p + partition_size, n))
              for p in range(0, max(n, 1), partition_size)]
    return merge_partitions(states)


def blockwise_softmax_sum(q, K, V, scale: float, block_size: int) -> np.ndarray:
    """P1 §1's second formula taken literally: the sum over blocks of each
    block's own softmax-weighted values.  Kept only as a negative reference."""
    n = K.shape[0]
    total = np.zeros(V.shape[-1])
    for b0 in range(0, n, block_size):
        total = total + attention(q, K[b0:b0 + block_size], V[b0:b0 + block_size], scale)
    return total



# ---------------------------------------------------------------------------
# 8-bit KV storage.  The pages advise storing KV in a lower precision to save
# memory (P1 §4: blocks in bfloat16 halve memory at a small accuracy cost;
# P1 §5 and P2 §5: quantisation and compression of the cache) without fixing
# a format.  Reading: K and V pools hold OCP FP8 E4M3 codes (1 sign bit, 4
# exponent bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal;
# 0x7F / 0xFF are NaN; no infinities; largest finite 448), one float32 scale
# per pool: value = decode(code) * scale.  Writing a float x stores
# encode(x / scale), the division done in float32 (the precision the kernel
# works in), rounded to the nearest code with ties to the even code and
# saturated at +-448.
# ---------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """Float64 values of E4M3 codes, from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = sign * (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    sub = sign * (man / 8.0) * 2.0 ** -6
    out = np.where(exp == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes of float values: nearest code, ties to the code with an even
    last bit, magnitudes above 448 saturated to 448, NaN to 0x7F."""
    v = np.asarray(x, dtype=np.float64)
    table = e4m3_decode(np.arange(0x7F, dtype=np.uint8))      # values of codes 0x00 .. 0x7E
    out = np.empty(v.shape, dtype=np.uint8)
    flat_v, flat_o = v.reshape(-1), out.reshape(-1)
    for i, xv in enumerate(flat_v):
        if np.isnan(xv):
            flat_o[i] = 0x7F
            continue
        a = min(abs(xv), 448.0)
        j = int(np.searchsorted(table, a))            # table[j-1] < a <= table[j]
        if j < len(table) and table[j] == a:
            code = j
        else:
            lo, hi = j - 1, j
            dl, dh = a - table[lo], table[hi] - a
            code = lo if dl < dh else hi if dh < dl else (lo if lo % 2 == 0 else hi)
        flat_o[i] = code | (0x80 if (xv < 0 or (xv == 0 and np.signbit(xv))) else 0)
    return out


def quantize_e4m3(x_f32, scale: float) -> np.ndarray:
    """Codes stored for float32 values ``x_f32`` with pool scale ``scale``:
    encode(float32(x) / float32(scale))."""
    q = np.asarray(x_f32, dtype=np.float32) / np.float32(scale)
    return e4m3_encode(q.astype(np.float64))


def cache_write_fp8(key_cache, value_cache, key, value, slot_mapping, block_size: int,
                    src_dtype: str, k_scale: float, v_scale: float) -> None:
    """The cache write of ``cache_write`` into E4M3 pools: each row is widened
    from its storage type to float32 and quantised with its pool's scale."""
    kq = quantize_e4m3(to_f64(key, src_dtype).astype(np.float32), k_scale)
    vq = quantize_e4m3(to_f64(value, src_dtype).astype(np.float32), v_scale)
    cache_write(key_cache, value_cache, kq, vq, slot_mapping, block_size)


def paged_decode_fp8(q, key_cache, value_cache, block_tables, context_lens, block_size: int,
                     scale: float, q_dtype: str, k_scale: float, v_scale: float,
                     num_kv_heads: int | None = None, pairs=None) -> np.ndarray:
    """``paged_decode`` over E4M3 pools: each (sequence, head) gathers its
    codes through the table, takes their values decode(code) * pool scale in
    float64, and attends."""
    q64 = to_f64(q, q_dtype)
    S, H, D = q64.shape
    Hkv = key_cache.shape[1] if num_kv_heads is None else num_kv_heads
    ks, vs = float(np.float32(k_scale)), float(np.float32(v_scale))
    out = np.full((S, H, D), np.nan)
    todo = pairs if pairs is not None else [(s, h) for s in range(S) for h in range(H)]
    for s, h in todo:
        n = int(context_lens[s])
        g = kv_head_of(h, H, Hkv)
        K = e4m3_decode(gather_context(key_cache, block_tables[s], n, g, block_size)) * ks
        V = e4m3_decode(gather_context(value_cache, block_tables[s], n, g, block_size)) * vs
        out[s, h] = attention(q64[s, h], K, V, scale)
    return out


def paged_prefill_fp8(q, key_cache, value_cache, block_tables, context_lens, query_start,
                      block_size: int, scale: float, q_dtype: str, k_scale: float,
                      v_scale: float, num_kv_heads: int | None = None, rows=None) -> np.ndarray:
    """``paged_prefill`` over E4M3 pools: query row j of sequence s (position
    p = ctx - qlen + j) gathers the codes of tokens 0..p through the table,
    takes their values decode(code) * pool scale in float64, and attends."""
    q64 = to_f64(q, q_dtype)
    T, H, D = q64.shape
    Hkv = key_cache.shape[1] if num_kv_heads is None else num_kv_heads
    ks, vs = float(np.float32(k_scale)), float(np.float32(v_scale))
    seq_of = np.full(T, -1, dtype=np.int64)
    for s in range(len(context_lens)):
        seq_of[int(query_start[s]):int(query_start[s + 1])] = s
    out = np.full((T, H, D), np.nan)
    todo = rows if rows is not None else [(i, h) for i in range(T) for h in range(H)]
    for i, h in todo:
        s = int(seq_of[i])
        qlen = int(query_start[s + 1]) - int(query_start[s])
        n = int(context_lens[s]) - qlen + (i - int(query_start[s])) + 1
        g = kv_head_of(h, H, Hkv)
        K = e4m3_decode(gather_context(key_cache, block_tables[s], n, g, block_size)) * ks
        V = e4m3_decode(gather_context(value_cache, block_tables[s], n, g, block_size)) * vs
        out[i, h] = attention(q64[i, h], K, V, scale)
    return out


# ---------------------------------------------------------------------------
# Byte accounting -- P2 §2.2: KV bytes = 2 x tokens x layers x heads x
# head_dim x element bytes.
# ---------------------------------------------------------------------------

def kv_cache_bytes(seq_len: int, num_layers: int, num_heads: int, head_dim: int,
                   dtype_size: int) -> int:
    return 2 * seq_len * num_layers * num_heads * head_dim * dtype_size
