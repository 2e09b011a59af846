"""GPU parity of pa_prefill (causal prompt attention through the block
table, on the matrix cores) against the oracle's paged_prefill."""
import sys

import numpy as np
import pytest
import torch

import oracle.blocks as OB
import oracle.paged as P
import tests._bounds as BD
import paged_kv_cache_368_amd as pa
from workloads import build, from_torch, normal_array, to_torch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()


def _case(dtype, ctx, qlens, H, Hkv, D, B, seed=11):
    """Pools, tables and query rows from the seeded generators (unused slots
    are NaN); the queries are the last qlen tokens of each context."""
    wl = build("prefill", dtype, ctx, H, Hkv, D, B, seed=seed, pool="choice", pool_factor=1.3,
               value_scale=0.5)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = normal_array(seed, 40, (int(qs[-1]), H, D), dtype, 0.5)
    return wl, qs, q


def _run(wl, qs, q, max_query_len=None, dev_tables=None):
    dt = wl.dtype
    T = q.shape[0]
    out = torch.full((T, wl.num_heads, wl.head_dim), float("inf"),
                     dtype=torch.float16 if dt == "f16" else torch.bfloat16, device="cuda")
    mq = int(np.diff(qs).max()) if max_query_len is None else max_query_len
    tables = wl.block_tables if dev_tables is None else dev_tables
    pa.pa_prefill(out, to_torch(q, dt, "cuda"), to_torch(wl.key_cache, dt, "cuda"),
                  to_torch(wl.value_cache, dt, "cuda"), torch.tensor(tables, device="cuda"),
                  torch.tensor(wl.context_lens, device="cuda"), torch.tensor(qs, device="cuda"),
                  mq, wl.max_context_len, wl.scale)
    torch.cuda.synchronize()
    return P.to_f64(from_torch(out, dt), dt)


def _oracle(wl, qs, q, rows=None):
    return P.paged_prefill(q, wl.key_cache, wl.value_cache, wl.block_tables, wl.context_lens, qs,
                           wl.block_size, wl.scale, wl.dtype, wl.num_kv_heads, rows)


CASES = [
    ("fresh_mha_d128", dict(ctx=[1, 16, 17, 100, 45], qlens=None, H=4, Hkv=4, D=128, B=16)),
    ("fresh_gqa_d64_b32", dict(ctx=[70, 33], qlens=None, H=8, Hkv=2, D=64, B=32)),
    ("suffix_mha_b64", dict(ctx=[200, 64, 300, 5], qlens=[37, 1, 64, 5], H=2, Hkv=2, D=128, B=64)),
    ("suffix_gqa_d128", dict(ctx=[129, 260], qlens=[40, 3], H=4, Hkv=1, D=128, B=16)),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(name, kw, dtype):
    _say(f"prefill {name} {dtype}")
    qlens = kw["qlens"] or kw["ctx"]
    wl, qs, q = _case(dtype, kw["ctx"], qlens, kw["H"], kw["Hkv"], kw["D"], kw["B"])
    got = _run(wl, qs, q)
    BD.assert_close(got, _oracle(wl, qs, q), dtype, name)


@pytest.mark.parametrize("scale", [0.0, -0.125, 2.0])
def test_prefill_other_scales(scale):
    """A zero scale (equal weights over each row's causal window: masked
    tokens must still count zero), a negative one and a large one."""
    _say(f"prefill scale {scale}")
    wl, qs, q = _case("f16", [40, 77, 16], [40, 30, 16], 2, 2, 128, 16, seed=14)
    wl.scale = scale
    got = _run(wl, qs, q)
    BD.assert_close(got, _oracle(wl, qs, q), "f16", f"scale {scale}")


def test_prefill_crosses_table_windows():
    """Contexts longer than one staged window of block ids (4096 tokens)."""
    _say("prefill long contexts across windows")
    ctx, qlens = [4100, 8200, 4096], [20, 3, 17]
    wl, qs, q = _case("bf16", ctx, qlens, 2, 1, 64, 16, seed=12)
    got = _run(wl, qs, q)
    BD.assert_close(got, _oracle(wl, qs, q), "bf16", "long contexts")


def test_prefill_one_query_row_is_decode():
    _say("prefill qlen=1 vs decode")
    ctx = [90, 257, 16]
    wl, qs, q = _case("f16", ctx, [1, 1, 1], 4, 4, 128, 16, seed=13)
    got = _run(wl, qs, q)
    out = torch.empty((3, 4, 128), dtype=torch.float16, device="cuda")
    dq, dk = to_torch(q, "f16", "cuda"), to_torch(wl.key_cache, "f16", "cuda")
    pa.pa_decode(out, dq, dk, to_torch(wl.value_cache, "f16", "cuda"),
                 torch.tensor(wl.block_tables, device="cuda"),
                 torch.tensor(wl.context_lens, device="cuda"), wl.max_context_len, wl.scale,
                 workspace=pa.decode_workspace(dq, dk, wl.max_context_len))
    torch.cuda.synchronize()
    dec = P.to_f64(from_torch(out, "f16"), "f16")
    BD.assert_close(got, dec, "f16", "prefill row vs decode")


def test_prefill_with_shared_prefix_blocks():
    """Two requests share a 48-token prefix (the same physical blocks, from
    the block manager's prefix sharing); each prefills only its own suffix."""
    _say("prefill shared prefix")
    B, H, Hkv, D, dt = 16, 4, 2, 128, "bf16"
    bm = OB.BlockManager(40, B)
    bm.allocate_for_request(1, 48 + 30)
    bm.share_prefix_blocks(1, 2, 48)
    for pos in range(48, 48 + 25):
        bm.append_slot(2, pos)
    tables = np.full((2, 5), -1, np.int32)
    for i, rid in enumerate((1, 2)):
        t = bm.table(rid)
        tables[i, :len(t)] = t
    ctx = np.array([78, 73], np.int32)
    wl = build("shared", dt, ctx, H, Hkv, D, B, seed=14, num_blocks=40)
    wl.key_cache = normal_array(14, 1, (40, Hkv, B, D), dt, 0.5)
    wl.value_cache = normal_array(14, 2, (40, Hkv, B, D), dt, 0.5)
    wl.block_tables = tables
    qs = np.array([0, 30, 55], np.int32)
    q = normal_array(14, 3, (55, H, D), dt, 0.5)
    got = _run(wl, qs, q)
    BD.assert_close(got, _oracle(wl, qs, q), dt, "shared prefix")


def test_prefill_invalid_values_poison_only_their_rows():
    _say("prefill invalid device values")
    ctx = [50, 60, 40]
    wl, qs, q = _case("f16", ctx, [10, 12, 8], 2, 2, 64, 16, seed=15)
    tables = wl.block_tables.copy()
    tables[1, 1] = wl.num_blocks + 9                      # bad id in sequence 1
    cl = wl.context_lens.copy()
    cl[2] = 5                                             # qlen 8 > context 5 in sequence 2
    wl.context_lens = cl
    got = _run(wl, qs, q, dev_tables=tables)
    assert np.isnan(got[qs[1]:qs[3]]).all()
    ref = _oracle(wl, qs, q, rows=[(i, h) for i in range(qs[0], qs[1]) for h in range(2)])
    BD.assert_close(got[:qs[1]], ref[:qs[1]], "f16", "good rows")


def test_prefill_empty_query_ranges():
    _say("prefill empty query ranges")
    ctx = [30, 20, 25]
    wl, qs, q = _case("bf16", ctx, [0, 7, 0], 2, 2, 128, 16, seed=16)
    got = _run(wl, qs, q)
    BD.assert_close(got, _oracle(wl, qs, q), "bf16", "empty ranges")


@pytest.mark.parametrize("prefix", [0, 1536])
def test_prefill_full_size_sampled(prefix):
    """The inputs and launch bench.py times (--op prefill): 8 LLaMA-7B-shaped
    fp16 prompts of 2048 tokens (32 heads of 128, blocks of 16), whole or
    the last 512 after a cached 1536-token prefix; sampled (row, head) pairs
    against the oracle: both ends of every 256-row tile of the first and
    last sequences, every sequence's first and last row, and random ones."""
    S, H, D, B, n = 8, 32, 128, 16, 2048
    L = n - prefix
    _say(f"prefill full size, prefix {prefix}")
    wl = build("llama7b_prefill_f16", "f16", [n] * S, H, H, D, B, seed=7, pool="permutation",
               value_scale=0.5)
    qs = np.arange(S + 1, dtype=np.int32) * L
    q = normal_array(7, 40, (S * L, H, D), "f16", 0.5)
    got = _run(wl, qs, q, max_query_len=L)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(70 + prefix)
    rows = set()
    for s in (0, S - 1):
        for t0 in range(0, L, 256):
            rows.update({(s * L + t0, int(rng.integers(H))),
                         (s * L + min(t0 + 255, L - 1), int(rng.integers(H)))})
    for s in range(S):
        rows.update({(s * L, int(rng.integers(H))), (s * L + L - 1, int(rng.integers(H)))})
    rows.update((int(rng.integers(S * L)), int(rng.integers(H))) for _ in range(48))
    rows = sorted(rows)
    ref = _oracle(wl, qs, q, rows)
    idx = tuple(np.array(rows).T)
    BD.assert_close(got[idx], ref[idx], "f16", f"prefill full size, prefix {prefix}")
