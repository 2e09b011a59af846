"""ctypes binding of libpa.so (include/pa.h), same entry-point names.

Argument marshalling only: shapes are read off the tensors, pointers and the
current HIP stream are passed through, and a non-OK status raises
``PaError``.  Every computation happens in the library's kernels; there is no
fallback.  PyTorch is imported first so that the HIP runtime it ships is the
one libpa.so binds to (both carry the soname libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY names another build of the same C ABI (the sanitizer tests load a
# CPU-only build of the host code through it); by default the in-tree libpa.so.
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_PKG, "libpa.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "pa.h")

(PA_OK, PA_ERR_INVALID_ARGUMENT, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE_TOO_SMALL, PA_ERR_HIP,
 PA_ERR_NO_BLOCKS, PA_ERR_UNKNOWN_REQUEST, PA_ERR_STATE) = range(8)
DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_lib = None


class PaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pa status {status}: {message}")
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Open libpa.so (built by ``paged_kv_cache_368_amd.build``); raises if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build it with `python -m paged_kv_cache_368_amd.build`")
    lib = ctypes.CDLL(p, mode=ctypes.RTLD_GLOBAL)
    c = ctypes
    st, i32, ptr, sz = c.c_int, c.c_int32, c.c_void_p, c.c_size_t
    lib.pa_compute_slots.argtypes = [ptr, ptr, i32, ptr, ptr, ptr, i32, i32, i32, i32, ptr]
    lib.pa_compute_slots.restype = st
    lib.pa_cache_write.argtypes = [ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, i32, c.c_int, ptr]
    lib.pa_cache_write.restype = st
    lib.pa_decode_partition_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, c.c_int]
    lib.pa_decode_partition_size.restype = i32
    lib.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, c.c_int]
    lib.pa_decode_workspace_size.restype = sz
    lib.pa_decode.argtypes = [ptr, ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, i32, i32, i32, i32,
                              c.c_float, i32, ptr, sz, c.c_int, ptr]
    lib.pa_decode.restype = st
    lib.pa_append_decode.argtypes = [ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32,
                                     i32, i32, i32, i32, c.c_float, i32, ptr, sz, c.c_int, ptr]
    lib.pa_append_decode.restype = st
    lib.pa_decode_noalloc.argtypes = [ptr, ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, i32, i32,
                                      i32, i32, c.c_float, i32, c.c_int, ptr]
    lib.pa_decode_noalloc.restype = st
    lib.pa_read_probe.argtypes = [ptr, c.c_int64, c.c_int64, ptr, ptr, ptr]
    lib.pa_read_probe.restype = st
    lib.pa_append_decode_fp8.argtypes = [ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, i32, i32, i32,
                                         i32, i32, i32, i32, i32, c.c_float, c.c_float,
                                         c.c_float, i32, ptr, sz, c.c_int, ptr]
    lib.pa_append_decode_fp8.restype = st
    f32 = c.c_float
    lib.pa_cache_write_fp8.argtypes = [ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, i32, c.c_int,
                                       f32, f32, ptr]
    lib.pa_cache_write_fp8.restype = st
    lib.pa_decode_fp8.argtypes = [ptr, ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, i32, i32, i32,
                                  i32, f32, f32, f32, i32, ptr, sz, c.c_int, ptr]
    lib.pa_decode_fp8.restype = st
    lib.pa_prefill.argtypes = [ptr, ptr, ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, i32, i32,
                               i32, i32, i32, i32, f32, c.c_int, ptr]
    lib.pa_prefill.restype = st
    lib.pa_prefill_fp8.argtypes = [ptr, ptr, ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, i32,
                                   i32, i32, i32, i32, i32, f32, f32, f32, c.c_int, ptr]
    lib.pa_prefill_fp8.restype = st
    lib.pa_copy_blocks.argtypes = [ptr, ptr, ptr, ptr, ptr, i32, c.c_int64, i32, i32, ptr]
    lib.pa_copy_blocks.restype = st
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = c.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = c.c_char_p
    # host block manager (include/pa_blocks.h)
    u64 = c.c_uint64
    for name, args in {
        "pa_bm_create": [i32, i32, ptr],
        "pa_bm_allocate": [ptr, u64, i32, ptr],
        "pa_bm_append_slot": [ptr, u64, i32, ptr, ptr, ptr, ptr],
        "pa_bm_append_slots": [ptr, ptr, ptr, i32, ptr, ptr, ptr, ptr],
        "pa_bm_share_prefix": [ptr, u64, u64, i32],
        "pa_bm_fork": [ptr, u64, u64],
        "pa_bm_free_request": [ptr, u64],
        "pa_bm_stats": [ptr, ptr, ptr, ptr],
        "pa_bm_table": [ptr, u64, ptr, i32, ptr],
        "pa_bm_free_ids": [ptr, ptr, i32, ptr],
        "pa_bm_fill_tables": [ptr, ptr, i32, i32, ptr],
    }.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = st
    lib.pa_bm_destroy.argtypes = [ptr]
    lib.pa_bm_destroy.restype = None
    lib.pa_bm_ref_count.argtypes = [ptr, i32]
    lib.pa_bm_ref_count.restype = i32
    if path is None:
        _lib = lib
    return lib


def declared_functions(headers=None) -> list[str]:
    """Names of the functions the headers under include/ declare."""
    if headers is None:
        inc = os.path.dirname(HEADER)
        headers = [os.path.join(inc, f) for f in sorted(os.listdir(inc)) if f.endswith(".h")]
    names = set()
    for header in headers:
        with open(header) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def _check(status: int) -> None:
    if status != PA_OK:
        raise PaError(status, load_library().pa_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _opt(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _workspace(workspace):
    """(pointer, bytes) of the caller's decode workspace, or (None, 0).  The
    library checks the size and refuses a split-context call without one."""
    if workspace is None:
        return None, 0
    _dev(workspace, "workspace")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def decode_workspace(q: torch.Tensor, key_cache: torch.Tensor, max_context_len: int,
                     partition_size: int = 0) -> torch.Tensor | None:
    """Allocate the device workspace that pa_decode / pa_append_decode (or
    their _fp8 forms, for uint8 pools) need for these inputs, or return None
    when they need none.  The decode calls themselves never allocate: a caller
    allocates this once and passes it to every call of that size or smaller."""
    S, H, D = q.shape
    _, Hkv, B, _ = key_cache.shape
    dt = torch.uint8 if key_cache.dtype == torch.uint8 else q.dtype
    n = pa_decode_workspace_size(S, H, Hkv, D, B, max_context_len, partition_size, dt)
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def pa_version() -> str:
    return load_library().pa_version().decode()


def pa_last_error() -> str:
    return load_library().pa_last_error().decode()


def pa_compute_slots(slot_mapping: torch.Tensor, block_tables: torch.Tensor, block_size: int,
                     num_blocks: int, context_lens: torch.Tensor | None = None,
                     seq_ids: torch.Tensor | None = None,
                     positions: torch.Tensor | None = None) -> torch.Tensor:
    """Fill int64 ``slot_mapping`` with the pool slot of each token."""
    lib = load_library()
    for n, t in (("slot_mapping", slot_mapping), ("block_tables", block_tables)):
        _dev(t, n)
    if slot_mapping.dtype != torch.int64 or block_tables.dtype != torch.int32:
        raise ValueError("slot_mapping must be int64 and block_tables int32")
    for n, t in (("context_lens", context_lens), ("seq_ids", seq_ids), ("positions", positions)):
        if t is not None:
            _dev(t, n)
            if t.dtype != torch.int32:
                raise ValueError(f"{n} must be int32")
    _check(lib.pa_compute_slots(
        ctypes.c_void_p(slot_mapping.data_ptr()), ctypes.c_void_p(block_tables.data_ptr()),
        block_tables.shape[1], _opt(context_lens), _opt(seq_ids), _opt(positions),
        slot_mapping.numel(), block_tables.shape[0], block_size, num_blocks, _stream(slot_mapping)))
    return slot_mapping


def pa_cache_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                   value_cache: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """Copy key/value [T][Hkv][D] into the pools [NB][Hkv][B][D] at their slots."""
    lib = load_library()
    for n, t in (("key", key), ("value", value), ("key_cache", key_cache),
                 ("value_cache", value_cache), ("slot_mapping", slot_mapping)):
        _dev(t, n)
    if key.dtype not in DTYPE_CODES or any(t.dtype != key.dtype for t in (value, key_cache, value_cache)):
        raise ValueError("key, value and the pools must share one of float32/float16/bfloat16")
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    NB, Hkv, B, D = key_cache.shape
    if tuple(value_cache.shape) != (NB, Hkv, B, D) or key.shape[1:] != (Hkv, D) or value.shape != key.shape:
        raise ValueError("shape mismatch between key/value and the pools")
    if slot_mapping.numel() != key.shape[0]:
        raise ValueError("slot_mapping must have one entry per token")
    _check(lib.pa_cache_write(
        ctypes.c_void_p(key.data_ptr()), ctypes.c_void_p(value.data_ptr()),
        ctypes.c_void_p(key_cache.data_ptr()), ctypes.c_void_p(value_cache.data_ptr()),
        ctypes.c_void_p(slot_mapping.data_ptr()), key.shape[0], Hkv, D, B, NB,
        DTYPE_CODES[key.dtype], _stream(key)))


def _mem(t: torch.Tensor, name: str) -> None:
    """A pool for pa_copy_blocks: a contiguous device tensor or a pinned host one."""
    if not isinstance(t, torch.Tensor) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor")
    if t.device.type != "cuda" and not t.is_pinned():
        raise ValueError(f"{name} must be a device tensor or pinned host memory")


def pa_copy_blocks(dst_key: torch.Tensor, src_key: torch.Tensor, block_pairs: torch.Tensor,
                   dst_value: torch.Tensor | None = None,
                   src_value: torch.Tensor | None = None) -> None:
    """Copy whole blocks ``dst[d] = src[s]`` for each (s, d) row of the device
    int32 ``block_pairs`` [n][2]; pools are [num_blocks][...] device tensors
    or pinned host tensors of one dtype.  Launches on the current stream."""
    lib = load_library()
    _dev(block_pairs, "block_pairs")
    if block_pairs.dtype != torch.int32 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be int32 [n][2]")
    pools = [("dst_key", dst_key), ("src_key", src_key)]
    if (dst_value is None) != (src_value is None):
        raise ValueError("give both dst_value and src_value, or neither")
    if dst_value is not None:
        pools += [("dst_value", dst_value), ("src_value", src_value)]
    for n, t in pools:
        _mem(t, n)
    block_bytes = src_key[0].numel() * src_key.element_size() if src_key.shape[0] else 0
    for n, t in pools:
        if t.element_size() * (t[0].numel() if t.shape[0] else 0) != block_bytes:
            raise ValueError(f"{n} has a different block size")
    _check(lib.pa_copy_blocks(
        ctypes.c_void_p(dst_key.data_ptr()), _opt(dst_value), ctypes.c_void_p(src_key.data_ptr()),
        _opt(src_value), ctypes.c_void_p(block_pairs.data_ptr()), block_pairs.shape[0],
        block_bytes, dst_key.shape[0], src_key.shape[0], _stream(block_pairs)))


PA_FP8_E4M3 = 3


def pa_cache_write_fp8(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                       value_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float,
                       v_scale: float) -> None:
    """Quantise key/value [T][Hkv][D] (f32/f16/bf16) into uint8 E4M3 pools
    [NB][Hkv][B][D] at their slots: code(x / scale)."""
    lib = load_library()
    for n, t in (("key", key), ("value", value), ("key_cache", key_cache),
                 ("value_cache", value_cache), ("slot_mapping", slot_mapping)):
        _dev(t, n)
    if key.dtype not in DTYPE_CODES or value.dtype != key.dtype:
        raise ValueError("key and value must share one of float32/float16/bfloat16")
    if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8:
        raise ValueError("E4M3 pools are uint8 tensors")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != key.shape[0]:
        raise ValueError("slot_mapping must be int64 with one entry per token")
    NB, Hkv, B, D = key_cache.shape
    if tuple(value_cache.shape) != (NB, Hkv, B, D) or key.shape[1:] != (Hkv, D) or value.shape != key.shape:
        raise ValueError("shape mismatch between key/value and the pools")
    _check(lib.pa_cache_write_fp8(
        ctypes.c_void_p(key.data_ptr()), ctypes.c_void_p(value.data_ptr()),
        ctypes.c_void_p(key_cache.data_ptr()), ctypes.c_void_p(value_cache.data_ptr()),
        ctypes.c_void_p(slot_mapping.data_ptr()), key.shape[0], Hkv, D, B, NB,
        DTYPE_CODES[key.dtype], float(k_scale), float(v_scale), _stream(key)))


def pa_decode_fp8(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                  value_cache: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor, max_context_len: int, k_scale: float,
                  v_scale: float, scale: float, partition_size: int = 0,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """PagedAttention decode over uint8 E4M3 pools (values code * scale) into
    ``out`` [S][H][D] of q's type (fp16/bf16); see include/pa.h."""
    lib = load_library()
    for n, t in (("out", out), ("q", q), ("key_cache", key_cache), ("value_cache", value_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens)):
        _dev(t, n)
    if q.dtype not in (torch.float16, torch.bfloat16) or out.dtype != q.dtype:
        raise ValueError("q and out must share float16 or bfloat16")
    if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8:
        raise ValueError("E4M3 pools are uint8 tensors")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    S, H, D = q.shape
    NB, Hkv, B, D2 = key_cache.shape
    if D2 != D or tuple(value_cache.shape) != (NB, Hkv, B, D) or tuple(out.shape) != (S, H, D):
        raise ValueError("shape mismatch between q, out and the pools")
    if block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables and context_lens must have one row per sequence")
    ws_ptr, ws_bytes = _workspace(workspace)
    _check(lib.pa_decode_fp8(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(key_cache.data_ptr()), ctypes.c_void_p(value_cache.data_ptr()),
        ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(context_lens.data_ptr()),
        S, H, Hkv, D, B, NB, block_tables.shape[1], max_context_len, float(scale), float(k_scale),
        float(v_scale), partition_size, ws_ptr, ws_bytes, DTYPE_CODES[q.dtype], _stream(q)))
    return out


def pa_prefill(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
               value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
               query_start: torch.Tensor, max_query_len: int, max_context_len: int,
               scale: float) -> torch.Tensor:
    """Paged prefill into ``out`` [T][H][D] for query rows ``q`` [T][H][D]
    (fp16/bf16); sequence s owns rows query_start[s] .. query_start[s+1]-1,
    the last tokens of its context; see include/pa.h."""
    lib = load_library()
    for n, t in (("out", out), ("q", q), ("key_cache", key_cache), ("value_cache", value_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens),
                 ("query_start", query_start)):
        _dev(t, n)
    if q.dtype not in (torch.float16, torch.bfloat16) or any(
            t.dtype != q.dtype for t in (out, key_cache, value_cache)):
        raise ValueError("q, out and the pools must share float16 or bfloat16")
    for n, t in (("block_tables", block_tables), ("context_lens", context_lens),
                 ("query_start", query_start)):
        if t.dtype != torch.int32:
            raise ValueError(f"{n} must be int32")
    T, H, D = q.shape
    NB, Hkv, B, D2 = key_cache.shape
    S = context_lens.numel()
    if D2 != D or tuple(value_cache.shape) != (NB, Hkv, B, D) or tuple(out.shape) != (T, H, D):
        raise ValueError("shape mismatch between q, out and the pools")
    if block_tables.shape[0] != S or query_start.numel() != S + 1:
        raise ValueError("block_tables needs one row and query_start S + 1 entries")
    _check(lib.pa_prefill(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(key_cache.data_ptr()), ctypes.c_void_p(value_cache.data_ptr()),
        ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(context_lens.data_ptr()),
        ctypes.c_void_p(query_start.data_ptr()), S, T, H, Hkv, D, B, NB, block_tables.shape[1],
        max_query_len, max_context_len, float(scale), DTYPE_CODES[q.dtype], _stream(q)))
    return out


def pa_prefill_fp8(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                   value_cache: torch.Tensor, block_tables: torch.Tensor,
                   context_lens: torch.Tensor, query_start: torch.Tensor, max_query_len: int,
                   max_context_len: int, k_scale: float, v_scale: float,
                   scale: float) -> torch.Tensor:
    """pa_prefill over uint8 E4M3 pools (values code * scale): query rows
    ``q`` [T][H][D] (fp16/bf16) into ``out``; see include/pa.h."""
    lib = load_library()
    for n, t in (("out", out), ("q", q), ("key_cache", key_cache), ("value_cache", value_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens),
                 ("query_start", query_start)):
        _dev(t, n)
    if q.dtype not in (torch.float16, torch.bfloat16) or out.dtype != q.dtype:
        raise ValueError("q and out must share float16 or bfloat16")
    if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8:
        raise ValueError("E4M3 pools are uint8 tensors")
    for n, t in (("block_tables", block_tables), ("context_lens", context_lens),
                 ("query_start", query_start)):
        if t.dtype != torch.int32:
            raise ValueError(f"{n} must be int32")
    T, H, D = q.shape
    NB, Hkv, B, D2 = key_cache.shape
    S = context_lens.numel()
    if D2 != D or tuple(value_cache.shape) != (NB, Hkv, B, D) or tuple(out.shape) != (T, H, D):
        raise ValueError("shape mismatch between q, out and the pools")
    if block_tables.shape[0] != S or query_start.numel() != S + 1:
        raise ValueError("block_tables needs one row and query_start S + 1 entries")
    _check(lib.pa_prefill_fp8(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(key_cache.data_ptr()), ctypes.c_void_p(value_cache.data_ptr()),
        ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(context_lens.data_ptr()),
        ctypes.c_void_p(query_start.data_ptr()), S, T, H, Hkv, D, B, NB, block_tables.shape[1],
        max_query_len, max_context_len, float(scale), float(k_scale), float(v_scale),
        DTYPE_CODES[q.dtype], _stream(q)))
    return out


def pa_decode_partition_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                             max_context_len, partition_size=0, dtype=torch.float16) -> int:
    return load_library().pa_decode_partition_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                   block_size, max_context_len, partition_size,
                                                   _size_dtype(dtype))


def pa_append_decode(out: torch.Tensor, q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                     key_cache: torch.Tensor, value_cache: torch.Tensor,
                     block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                     scale: float, partition_size: int = 0,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step in one launch: writes each sequence's newest token
    (position context_lens - 1; rows ``key``/``value`` [S][Hkv][D]) into its
    slot and runs decode into ``out``; see include/pa.h."""
    lib = load_library()
    for n, t in (("out", out), ("q", q), ("key", key), ("value", value),
                 ("key_cache", key_cache), ("value_cache", value_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens)):
        _dev(t, n)
    if q.dtype not in DTYPE_CODES or any(t.dtype != q.dtype
                                         for t in (out, key, value, key_cache, value_cache)):
        raise ValueError("q, out, key, value and the pools must share one of "
                         "float32/float16/bfloat16")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    S, H, D = q.shape
    NB, Hkv, B, D2 = key_cache.shape
    if D2 != D or tuple(value_cache.shape) != (NB, Hkv, B, D) or tuple(out.shape) != (S, H, D):
        raise ValueError("shape mismatch between q, out and the pools")
    if tuple(key.shape) != (S, Hkv, D) or tuple(value.shape) != (S, Hkv, D):
        raise ValueError("key and value must be [num_seqs][num_kv_heads][head_dim]")
    if block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables and context_lens must have one row per sequence")
    ws_ptr, ws_bytes = _workspace(workspace)
    _check(lib.pa_append_decode(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(key.data_ptr()), ctypes.c_void_p(value.data_ptr()),
        ctypes.c_void_p(key_cache.data_ptr()), ctypes.c_void_p(value_cache.data_ptr()),
        ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(context_lens.data_ptr()),
        S, H, Hkv, D, B, NB, block_tables.shape[1], max_context_len, float(scale),
        partition_size, ws_ptr, ws_bytes, DTYPE_CODES[q.dtype], _stream(q)))
    return out


def pa_append_decode_fp8(out: torch.Tensor, q: torch.Tensor, key: torch.Tensor,
                         value: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor,
                         max_context_len: int, k_scale: float, v_scale: float,
                         scale: float, partition_size: int = 0,
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """pa_append_decode over E4M3 pools (uint8 codes, value = code * scale):
    the newest token's rows (``key``/``value`` [S][Hkv][D], q's type) are
    quantised into their slot and attended; see include/pa.h."""
    lib = load_library()
    for n, t in (("out", out), ("q", q), ("key", key), ("value", value),
                 ("key_cache", key_cache), ("value_cache", value_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens)):
        _dev(t, n)
    if q.dtype not in (torch.float16, torch.bfloat16) or any(
            t.dtype != q.dtype for t in (out, key, value)):
        raise ValueError("q, out, key and value must share float16 or bfloat16")
    if key_cache.dtype != torch.uint8 or value_cache.dtype != torch.uint8:
        raise ValueError("E4M3 pools are uint8 tensors of codes")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    S, H, D = q.shape
    NB, Hkv, B, D2 = key_cache.shape
    if D2 != D or tuple(value_cache.shape) != (NB, Hkv, B, D) or tuple(out.shape) != (S, H, D):
        raise ValueError("shape mismatch between q, out and the pools")
    if tuple(key.shape) != (S, Hkv, D) or tuple(value.shape) != (S, Hkv, D):
        raise ValueError("key and value must be [num_seqs][num_kv_heads][head_dim]")
    if block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables and context_lens must have one row per sequence")
    ws_ptr, ws_bytes = _workspace(workspace)
    _check(lib.pa_append_decode_fp8(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(key.data_ptr()), ctypes.c_void_p(value.data_ptr()),
        ctypes.c_void_p(key_cache.data_ptr()), ctypes.c_void_p(value_cache.data_ptr()),
        ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(context_lens.data_ptr()),
        S, H, Hkv, D, B, NB, block_tables.shape[1], max_context_len, float(scale),
        float(k_scale), float(v_scale), partition_size, ws_ptr, ws_bytes,
        DTYPE_CODES[q.dtype], _stream(q)))
    return out


PA_READ_PROBE_SINK_WORDS = 2048


def pa_read_probe(buf: torch.Tensor, tile_bytes: int, order: torch.Tensor | None,
                  sink: torch.Tensor) -> torch.Tensor:
    """Read ``buf`` as tiles of ``tile_bytes`` in ``order`` (int32 tile
    indices; None: index order) with the library's read probe; returns the
    sink (one uint32 fold per work-group).  The caller times the call."""
    lib = load_library()
    _dev(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    if tile_bytes <= 0 or tile_bytes % 1024:
        raise ValueError("tile_bytes must be a positive multiple of 1024")
    n = nbytes // tile_bytes
    if order is not None:
        _dev(order, "order")
        if order.dtype != torch.int32 or order.numel() != n:
            raise ValueError("order must be int32 with one entry per tile")
    _dev(sink, "sink")
    if sink.numel() * sink.element_size() < PA_READ_PROBE_SINK_WORDS * 4:
        raise ValueError(f"sink must hold {PA_READ_PROBE_SINK_WORDS} 32-bit words")
    _check(lib.pa_read_probe(ctypes.c_void_p(buf.data_ptr()), tile_bytes, n,
                             ctypes.c_void_p(order.data_ptr()) if order is not None else None,
                             ctypes.c_void_p(sink.data_ptr()), _stream(buf)))
    return sink


def _size_dtype(dtype) -> int:
    """dtype code of the sizing functions: a torch float type, or torch.uint8
    (or PA_FP8_E4M3) for E4M3 pools."""
    if dtype == torch.uint8 or dtype == PA_FP8_E4M3:
        return PA_FP8_E4M3
    return DTYPE_CODES[dtype]


def pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                             max_context_len, partition_size=0, dtype=torch.float16) -> int:
    n = load_library().pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                block_size, max_context_len, partition_size,
                                                _size_dtype(dtype))
    if n == ctypes.c_size_t(-1).value:
        raise PaError(PA_ERR_INVALID_ARGUMENT, pa_last_error())
    return n


def pa_decode(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
              value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
              max_context_len: int, scale: float, partition_size: int = 0,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """PagedAttention decode into ``out`` [S][H][D]; see include/pa.h.

    ``workspace``: uint8 device memory of >= pa_decode_workspace_size bytes
    (``decode_workspace`` allocates one), or None when that size is 0.
    """
    lib = load_library()
    for n, t in (("out", out), ("q", q), ("key_cache", key_cache), ("value_cache", value_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens)):
        _dev(t, n)
    if q.dtype not in DTYPE_CODES or any(t.dtype != q.dtype for t in (out, key_cache, value_cache)):
        raise ValueError("q, out and the pools must share one of float32/float16/bfloat16")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    S, H, D = q.shape
    NB, Hkv, B, D2 = key_cache.shape
    if D2 != D or tuple(value_cache.shape) != (NB, Hkv, B, D) or tuple(out.shape) != (S, H, D):
        raise ValueError("shape mismatch between q, out and the pools")
    if block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables and context_lens must have one row per sequence")
    dt = DTYPE_CODES[q.dtype]
    ws_ptr, ws_bytes = _workspace(workspace)
    _check(lib.pa_decode(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(key_cache.data_ptr()), ctypes.c_void_p(value_cache.data_ptr()),
        ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(context_lens.data_ptr()),
        S, H, Hkv, D, B, NB, block_tables.shape[1], max_context_len, float(scale),
        partition_size, ws_ptr, ws_bytes, dt, _stream(q)))
    return out


PA_NOALLOC_SCRATCH_BYTES = 16 << 20


def pa_decode_noalloc(out: torch.Tensor, q: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, block_tables: torch.Tensor,
                      context_lens: torch.Tensor, max_context_len: int, scale: float,
                      partition_size: int = 0) -> torch.Tensor:
    """pa_decode without a workspace: split-context partials go to the
    library's static per-GPU scratch (PA_NOALLOC_SCRATCH_BYTES); see
    include/pa.h.  Calls that overlap on one GPU race on that scratch."""
    lib = load_library()
    for n, t in (("out", out), ("q", q), ("key_cache", key_cache), ("value_cache", value_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens)):
        _dev(t, n)
    if q.dtype not in DTYPE_CODES or any(t.dtype != q.dtype for t in (out, key_cache, value_cache)):
        raise ValueError("q, out and the pools must share one of float32/float16/bfloat16")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    S, H, D = q.shape
    NB, Hkv, B, D2 = key_cache.shape
    if D2 != D or tuple(value_cache.shape) != (NB, Hkv, B, D) or tuple(out.shape) != (S, H, D):
        raise ValueError("shape mismatch between q, out and the pools")
    if block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables and context_lens must have one row per sequence")
    _check(lib.pa_decode_noalloc(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(key_cache.data_ptr()), ctypes.c_void_p(value_cache.data_ptr()),
        ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(context_lens.data_ptr()),
        S, H, Hkv, D, B, NB, block_tables.shape[1], max_context_len, float(scale),
        partition_size, DTYPE_CODES[q.dtype], _stream(q)))
    return out
