"""GPU check of pa_read_probe (the read-bandwidth probe bench.py reports
beside the decode roofline): every tile is read exactly once, in index or
permuted order, so the XOR of all sink words equals the XOR of the buffer."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_368_amd as pa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load_library()


# Piece counts below, at (2 KiB x 65536) and above waves x 16 = 8192 x 16:
# each wave takes whole sixteen-piece batches, the last one with pieces a
# partial share, the waves after it none.
@pytest.mark.parametrize("tile_kib,tiles", [(4, 1), (4, 3001), (1, 777), (16, 64), (4, 33333),
                                            (2, 65536)])
def test_read_probe_reads_every_word_once(tile_kib, tiles):
    print(f"[case] read probe {tile_kib} KiB x {tiles}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(tiles)
    host = rng.integers(0, 2**32, size=tile_kib * 256 * tiles, dtype=np.uint32)
    want = int(np.bitwise_xor.reduce(host))
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    for order in (None, torch.from_numpy(rng.permutation(tiles).astype(np.int32)).cuda()):
        # Every work-group overwrites its word, those left without pieces too.
        sink = torch.from_numpy(rng.integers(-2**31, 2**31, size=pa.PA_READ_PROBE_SINK_WORDS,
                                             dtype=np.int32)).cuda()
        pa.pa_read_probe(buf, tile_kib * 1024, order, sink)
        torch.cuda.synchronize()
        got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
        assert got == want, f"order={'perm' if order is not None else 'index'}: {got:#x} != {want:#x}"
