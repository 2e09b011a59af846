"""Python binding of the host block manager (include/pa_blocks.h).

Marshalling only: every operation runs in libpa.so's C++ manager, which owns
its state; a non-OK status raises ``PaError`` with the library's message.
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._capi import PaError, load_library

_i32, _i64 = ctypes.c_int32, ctypes.c_int64


def _check(status: int) -> None:
    if status != 0:
        raise PaError(status, load_library().pa_last_error().decode())


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


class BlockManager:
    """A pool of ``num_blocks`` KV blocks of ``block_size`` tokens with
    per-request block tables (P3 §3), prefix sharing and beam forks (P3 §4)."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.pa_bm_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def allocate(self, request_id: int, num_tokens: int) -> int:
        n = _i32()
        _check(self._lib.pa_bm_allocate(self._h, request_id, num_tokens, ctypes.byref(n)))
        return n.value

    def append_slot(self, request_id: int, position: int):
        """-> (slot, new_block or None, (src, dst) or None)"""
        slot, nb, cs, cd = _i64(), _i32(), _i32(), _i32()
        _check(self._lib.pa_bm_append_slot(self._h, request_id, position, ctypes.byref(slot),
                                           ctypes.byref(nb), ctypes.byref(cs), ctypes.byref(cd)))
        return (slot.value, None if nb.value < 0 else nb.value,
                None if cs.value < 0 else (cs.value, cd.value))

    def append_slots(self, request_ids, positions):
        """Batched append for one decode step -> (slots int64 [n], copy pairs int32 [k][2])."""
        rids = np.ascontiguousarray(request_ids, dtype=np.uint64)
        pos = np.ascontiguousarray(positions, dtype=np.int32)
        n = len(rids)
        slots = np.empty(n, dtype=np.int64)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        nc, nd = _i32(), _i32()
        st = self._lib.pa_bm_append_slots(self._h, _ptr(rids), _ptr(pos), n, _ptr(slots),
                                          _ptr(pairs), ctypes.byref(nc), ctypes.byref(nd))
        if st != 0:
            err = PaError(st, self._lib.pa_last_error().decode())
            err.num_done = nd.value
            raise err
        return slots, pairs[:nc.value].copy()

    def share_prefix(self, src: int, dst: int, shared_len: int) -> None:
        _check(self._lib.pa_bm_share_prefix(self._h, src, dst, shared_len))

    def fork(self, src: int, dst: int) -> None:
        _check(self._lib.pa_bm_fork(self._h, src, dst))

    def free_request(self, request_id: int) -> None:
        _check(self._lib.pa_bm_free_request(self._h, request_id))

    def stats(self):
        """-> (free blocks, allocated blocks, live requests)"""
        f, a, r = _i32(), _i32(), _i32()
        _check(self._lib.pa_bm_stats(self._h, ctypes.byref(f), ctypes.byref(a), ctypes.byref(r)))
        return f.value, a.value, r.value

    def num_free(self) -> int:
        return self.stats()[0]

    def usage_ratio(self) -> float:
        return self.stats()[1] / self.num_blocks

    def ref_count(self, block_id: int) -> int:
        return self._lib.pa_bm_ref_count(self._h, block_id)

    def table(self, request_id: int) -> list[int]:
        n = _i32()
        buf = np.empty(max(self.num_blocks, 1), dtype=np.int32)
        _check(self._lib.pa_bm_table(self._h, request_id, _ptr(buf), len(buf), ctypes.byref(n)))
        return buf[:n.value].tolist()

    def free_ids(self) -> list[int]:
        n = _i32()
        buf = np.empty(self.num_blocks, dtype=np.int32)
        _check(self._lib.pa_bm_free_ids(self._h, _ptr(buf), len(buf), ctypes.byref(n)))
        return buf[:n.value].tolist()

    def fill_tables(self, request_ids, max_blocks_per_seq: int) -> np.ndarray:
        """Host int32 [len(request_ids)][max_blocks_per_seq], -1 padded."""
        rids = np.ascontiguousarray(request_ids, dtype=np.uint64)
        out = np.empty((len(rids), max_blocks_per_seq), dtype=np.int32)
        _check(self._lib.pa_bm_fill_tables(self._h, _ptr(rids), len(rids), max_blocks_per_seq,
                                           _ptr(out)))
        return out
