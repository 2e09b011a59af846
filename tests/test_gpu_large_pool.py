"""GPU parity on pools larger than 4 GiB each.

A serving pool on one 288 GB device holds far more than 2^32 bytes per
layer, so block ids reach byte offsets past 2^31 and 2^32 (and element
offsets past 2^31 for 16-bit types).  Each case here allocates K and V pools
of at least 4.5 GiB on the device, fills them with NaN, and places the blocks
the tables use on both sides of those boundaries and at the very end of the
pool.  Only the used blocks are generated on the host: the oracle runs on a
compact pool of those blocks with the tables renumbered into it (the output
does not depend on which physical ids hold the tiles, P3 §3), and the device
pools get the same tiles at their real ids.

Bars as in the other parity suites: bit-exact for slots, cache writes and
block copies; max(2e-3, 1 ulp) for 16-bit attention outputs, 1e-5 for fp32.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.paged as P
import tests._bounds as BD
import paged_kv_cache_368_amd as pa
from workloads import e4m3_codes, from_torch, nan_bits, normal_array, to_torch

pytestmark = pytest.mark.gpu

GIB = 1 << 30
POOL_BYTES = 4 * GIB + GIB // 2
ELEM = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class BigPools:
    """Device pools of >= 4.5 GiB and the compact host copy of their used
    blocks.  ``ids[c]`` is the device block id of compact block c."""

    def __init__(self, pool_dtype, Hkv, B, D, ctx, seed, extra_blocks=0):
        self.pool_dtype, self.Hkv, self.B, self.D = pool_dtype, Hkv, B, D
        self.ctx = np.asarray(ctx, dtype=np.int32)
        block_bytes = Hkv * B * D * ELEM[pool_dtype]
        self.NB = -(-POOL_BYTES // block_bytes)
        nblk = [-(-int(n) // B) for n in self.ctx]
        n_used = sum(nblk) + extra_blocks
        rng = np.random.default_rng(seed)
        # ids whose tiles start just below and above 2^31 and 2^32 bytes, the
        # last ids of the pool, and random ids from the upper half
        edge = []
        for bound in (1 << 31, 1 << 32):
            b0 = bound // block_bytes
            edge += list(range(b0 - 2, b0 + 3))
        edge += list(range(self.NB - 4, self.NB))
        rest = rng.choice(np.arange(self.NB // 2, self.NB - 4), n_used, replace=False)
        pool_ids = list(dict.fromkeys(edge + [int(x) for x in rest if int(x) not in edge]))
        self.ids = np.array(pool_ids[:n_used], dtype=np.int64)
        rng.shuffle(self.ids)
        assert len(self.ids) == n_used and self.ids.max() < self.NB
        assert int(self.ids.max()) * block_bytes >= 1 << 32
        MB = max(nblk) + 1
        self.ctables = np.full((len(self.ctx), MB), -1, np.int32)    # into the compact pool
        c = 0
        for s, k in enumerate(nblk):
            self.ctables[s, :k] = np.arange(c, c + k)
            c += k
        self.free_compact = list(range(c, n_used))                     # the extra blocks
        self.tables = np.where(self.ctables >= 0, self.ids[np.maximum(self.ctables, 0)],
                               -1).astype(np.int32)
        shape = (n_used, Hkv, B, D)
        if pool_dtype == "fp8":
            self.kc = e4m3_codes(seed, 2, shape)
            self.vc = e4m3_codes(seed, 3, shape)
        else:
            self.kc = normal_array(seed, 2, shape, pool_dtype)
            self.vc = normal_array(seed, 3, shape, pool_dtype)
        # slots past each context in its last block hold NaN
        for s, n in enumerate(self.ctx):
            if n % B:
                blk = self.ctables[s, n // B]
                self.kc[blk, :, n % B:, :] = nan_bits(pool_dtype)
                self.vc[blk, :, n % B:, :] = nan_bits(pool_dtype)
        self.k_dev = self._device_pool(self.kc)
        self.v_dev = self._device_pool(self.vc)
        self.tables_dev = torch.from_numpy(self.tables).cuda()
        self.ctx_dev = torch.from_numpy(self.ctx).cuda()

    def _device_pool(self, compact):
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "fp8": torch.uint8}[self.pool_dtype]
        pool = torch.empty((self.NB, self.Hkv, self.B, self.D), dtype=tdt, device="cuda")
        assert pool.numel() * pool.element_size() >= POOL_BYTES
        if self.pool_dtype == "fp8":
            pool.fill_(0x7F)
        else:
            pool.fill_(float("nan"))
        ids = torch.from_numpy(self.ids).cuda()
        pool.index_copy_(0, ids, to_torch(compact, self.pool_dtype, "cuda"))
        return pool

    def used_blocks(self, pool):
        """The used blocks of a device pool, in compact order, as raw words."""
        return from_torch(pool.index_select(0, torch.from_numpy(self.ids).cuda()),
                          self.pool_dtype)

    def max_ctx(self):
        return int(self.ctx.max())


@pytest.mark.parametrize("dtype,H,Hkv,D,B,ps", [
    ("f16", 8, 8, 128, 16, 0),          # vector kernel, one partition
    ("f16", 8, 8, 128, 16, 256),        # split contexts and the merge
    ("f32", 4, 4, 64, 32, 0),
    ("bf16", 32, 4, 128, 16, 0),        # grouped query heads on the matrix cores
    ("bf16", 16, 2, 64, 64, 512),
])
def test_decode_on_pool_beyond_4gib(dtype, H, Hkv, D, B, ps):
    _say(f"large-pool decode {dtype} H={H}/{Hkv} D={D} B={B} P={ps}")
    bp = BigPools(dtype, Hkv, B, D, [1, 37, 300, 1100, 2049], seed=900 + D + B)
    S = len(bp.ctx)
    q_raw = normal_array(901, 1, (S, H, D), dtype)
    q = to_torch(q_raw, dtype, "cuda")
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(D)
    pa.pa_decode(out, q, bp.k_dev, bp.v_dev, bp.tables_dev, bp.ctx_dev, bp.max_ctx(), scale, ps,
                 workspace=pa.decode_workspace(q, bp.k_dev, bp.max_ctx(), ps))
    torch.cuda.synchronize()
    ref = P.paged_decode(q_raw, bp.kc, bp.vc, bp.ctables, bp.ctx, B, scale, dtype, Hkv)
    got = P.to_f64(from_torch(out, dtype), dtype)
    BD.assert_close(got, ref, dtype, "decode on a pool beyond 4 GiB")


@pytest.mark.parametrize("dtype,H,Hkv", [("f16", 8, 8), ("bf16", 32, 4)])
def test_slots_write_and_append_on_pool_beyond_4gib(dtype, H, Hkv):
    """Slot resolution, the cache write and the one-launch step, each against
    the oracle on the compact pool: slots and pools bit-exact, outputs within
    the tolerance."""
    D, B = 128, 16
    _say(f"large-pool slots/cache_write/append {dtype} H={H}/{Hkv}")
    bp = BigPools(dtype, Hkv, B, D, [5, 16, 250, 1000], seed=910 + H)
    S = len(bp.ctx)
    # slots of every context token, resolved on the device through the real tables
    seq_ids = np.repeat(np.arange(S, dtype=np.int32), bp.ctx)
    positions = np.concatenate([np.arange(n, dtype=np.int32) for n in bp.ctx])
    slots = torch.empty(len(seq_ids), dtype=torch.int64, device="cuda")
    pa.pa_compute_slots(slots, bp.tables_dev, B, bp.NB, seq_ids=torch.from_numpy(seq_ids).cuda(),
                        positions=torch.from_numpy(positions).cuda())
    ref_slots = P.compute_slots(bp.tables, B, bp.NB, seq_ids=seq_ids, positions=positions)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)

    # overwrite the rows of every 3rd context token through those slots
    pick = np.arange(0, len(seq_ids), 3)
    key = normal_array(911, 4, (len(pick), Hkv, D), dtype)
    val = normal_array(911, 5, (len(pick), Hkv, D), dtype)
    pa.pa_cache_write(to_torch(key, dtype, "cuda"), to_torch(val, dtype, "cuda"), bp.k_dev,
                      bp.v_dev, slots[torch.from_numpy(pick).cuda()].contiguous())
    cslots = P.compute_slots(bp.ctables, B, len(bp.ids), seq_ids=seq_ids, positions=positions)[pick]
    P.cache_write(bp.kc, bp.vc, key, val, cslots, B)
    torch.cuda.synchronize()
    assert bp.used_blocks(bp.k_dev).tobytes() == bp.kc.tobytes()
    assert bp.used_blocks(bp.v_dev).tobytes() == bp.vc.tobytes()

    # one decode step: the newest token of each sequence written and attended
    ctx1 = bp.ctx.copy()
    q_raw = normal_array(912, 1, (S, H, D), dtype)
    nk = normal_array(912, 6, (S, Hkv, D), dtype)
    nv = normal_array(912, 7, (S, Hkv, D), dtype)
    q = to_torch(q_raw, dtype, "cuda")
    out = torch.empty_like(q)
    pa.pa_append_decode(out, q, to_torch(nk, dtype, "cuda"), to_torch(nv, dtype, "cuda"),
                        bp.k_dev, bp.v_dev, bp.tables_dev, bp.ctx_dev, bp.max_ctx(),
                        1.0 / math.sqrt(D), 0,
                        workspace=pa.decode_workspace(q, bp.k_dev, bp.max_ctx(), 0))
    torch.cuda.synchronize()
    new_slots = P.compute_slots(bp.ctables, B, len(bp.ids), context_lens=ctx1)
    P.cache_write(bp.kc, bp.vc, nk, nv, new_slots, B)
    assert bp.used_blocks(bp.k_dev).tobytes() == bp.kc.tobytes()
    assert bp.used_blocks(bp.v_dev).tobytes() == bp.vc.tobytes()
    ref = P.paged_decode(q_raw, bp.kc, bp.vc, bp.ctables, ctx1, B, 1.0 / math.sqrt(D), dtype, Hkv)
    BD.assert_close(P.to_f64(from_torch(out, dtype), dtype), ref, dtype, "append on a big pool")


@pytest.mark.parametrize("qt,H,Hkv", [("f16", 8, 8), ("bf16", 32, 4)])
def test_fp8_write_and_decode_on_pool_beyond_4gib(qt, H, Hkv):
    """E4M3 pools of >= 4.5 GiB: the quantising cache write bit-exact, decode
    (vector kernel for one query head per kv head, matrix cores otherwise)
    within the tolerance, and the one-launch step."""
    D, B = 128, 16
    ks, vs = 0.0625, 0.125
    _say(f"large-pool fp8 {qt} H={H}/{Hkv}")
    bp = BigPools("fp8", Hkv, B, D, [3, 40, 700, 1300], seed=920 + H)
    S = len(bp.ctx)
    seq_ids = np.repeat(np.arange(S, dtype=np.int32), bp.ctx)
    positions = np.concatenate([np.arange(n, dtype=np.int32) for n in bp.ctx])
    pick = np.arange(1, len(seq_ids), 5)
    slots = P.compute_slots(bp.tables, B, bp.NB, seq_ids=seq_ids[pick], positions=positions[pick])
    cslots = P.compute_slots(bp.ctables, B, len(bp.ids), seq_ids=seq_ids[pick],
                             positions=positions[pick])
    key = normal_array(921, 4, (len(pick), Hkv, D), qt)
    val = normal_array(921, 5, (len(pick), Hkv, D), qt)
    pa.pa_cache_write_fp8(to_torch(key, qt, "cuda"), to_torch(val, qt, "cuda"), bp.k_dev, bp.v_dev,
                          torch.from_numpy(slots).cuda(), ks, vs)
    P.cache_write_fp8(bp.kc, bp.vc, key, val, cslots, B, qt, ks, vs)
    torch.cuda.synchronize()
    assert bp.used_blocks(bp.k_dev).tobytes() == bp.kc.tobytes()
    assert bp.used_blocks(bp.v_dev).tobytes() == bp.vc.tobytes()

    q_raw = normal_array(922, 1, (S, H, D), qt)
    q = to_torch(q_raw, qt, "cuda")
    scale = 1.0 / math.sqrt(D)
    for ps in (0, 512):
        out = torch.empty_like(q)
        pa.pa_decode_fp8(out, q, bp.k_dev, bp.v_dev, bp.tables_dev, bp.ctx_dev, bp.max_ctx(),
                         ks, vs, scale, ps,
                         workspace=pa.decode_workspace(q, bp.k_dev, bp.max_ctx(), ps))
        torch.cuda.synchronize()
        ref = P.paged_decode_fp8(q_raw, bp.kc, bp.vc, bp.ctables, bp.ctx, B, scale, qt, ks, vs, Hkv)
        BD.assert_close(P.to_f64(from_torch(out, qt), qt), ref, qt, f"fp8 decode P={ps}")

    nk = normal_array(923, 6, (S, Hkv, D), qt)
    nv = normal_array(923, 7, (S, Hkv, D), qt)
    out = torch.empty_like(q)
    pa.pa_append_decode_fp8(out, q, to_torch(nk, qt, "cuda"), to_torch(nv, qt, "cuda"), bp.k_dev,
                            bp.v_dev, bp.tables_dev, bp.ctx_dev, bp.max_ctx(), ks, vs, scale, 0,
                            workspace=pa.decode_workspace(q, bp.k_dev, bp.max_ctx(), 0))
    torch.cuda.synchronize()
    new_slots = P.compute_slots(bp.ctables, B, len(bp.ids), context_lens=bp.ctx)
    P.cache_write_fp8(bp.kc, bp.vc, nk, nv, new_slots, B, qt, ks, vs)
    assert bp.used_blocks(bp.k_dev).tobytes() == bp.kc.tobytes()
    assert bp.used_blocks(bp.v_dev).tobytes() == bp.vc.tobytes()
    ref = P.paged_decode_fp8(q_raw, bp.kc, bp.vc, bp.ctables, bp.ctx, B, scale, qt, ks, vs, Hkv)
    BD.assert_close(P.to_f64(from_torch(out, qt), qt), ref, qt, "fp8 append on a big pool")


@pytest.mark.parametrize("dtype,H,Hkv", [("f16", 4, 4), ("bf16", 8, 2)])
def test_prefill_on_pool_beyond_4gib(dtype, H, Hkv):
    D, B = 128, 16
    _say(f"large-pool prefill {dtype} H={H}/{Hkv}")
    bp = BigPools(dtype, Hkv, B, D, [20, 300, 700], seed=930 + H)
    qlen = np.array([20, 300, 130], dtype=np.int32)       # the last 130 of the third: cached prefix
    qs = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    T = int(qs[-1])
    q_raw = normal_array(931, 1, (T, H, D), dtype)
    q = to_torch(q_raw, dtype, "cuda")
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(D)
    pa.pa_prefill(out, q, bp.k_dev, bp.v_dev, bp.tables_dev, bp.ctx_dev,
                  torch.from_numpy(qs).cuda(), int(qlen.max()), bp.max_ctx(), scale)
    torch.cuda.synchronize()
    ref = P.paged_prefill(q_raw, bp.kc, bp.vc, bp.ctables, bp.ctx, qs, B, scale, dtype, Hkv)
    BD.assert_close(P.to_f64(from_torch(out, dtype), dtype), ref, dtype, "prefill on a big pool")


def test_copy_blocks_on_pool_beyond_4gib():
    """Copy on write between blocks on both sides of the 2^31 and 2^32 byte
    offsets: bit-exact, and no other used block changes."""
    dtype, Hkv, B, D = "bf16", 8, 16, 128
    _say("large-pool copy_blocks")
    bp = BigPools(dtype, Hkv, B, D, [64, 200, 600], seed=940, extra_blocks=12)
    rng = np.random.default_rng(941)
    used = [c for c in range(len(bp.ids)) if c not in bp.free_compact]
    src_c = rng.choice(used, 12, replace=False)
    dst_c = np.array(bp.free_compact[:12])
    pairs_c = np.stack([src_c, dst_c], axis=1)
    pairs = bp.ids[pairs_c].astype(np.int32)
    pa.pa_copy_blocks(bp.k_dev, bp.k_dev, torch.from_numpy(pairs).cuda(), bp.v_dev, bp.v_dev)
    P.copy_blocks(bp.kc, bp.kc, pairs_c)
    P.copy_blocks(bp.vc, bp.vc, pairs_c)
    torch.cuda.synchronize()
    assert bp.used_blocks(bp.k_dev).tobytes() == bp.kc.tobytes()
    assert bp.used_blocks(bp.v_dev).tobytes() == bp.vc.tobytes()
