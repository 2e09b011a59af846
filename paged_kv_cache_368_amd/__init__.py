"""Paged KV-cache decode for AMD Instinct MI355X (gfx950).

The compute lives in libpa.so (hand-written HIP kernels behind the C ABI of
include/pa.h); this package is its thin Python binding, plus helpers that move
the seeded synthetic workloads onto the GPU.
"""
from ._capi import (  # noqa: F401
    DTYPE_CODES,
    LIB_PATH,
    PaError,
    declared_functions,
    decode_workspace,
    load_library,
    PA_FP8_E4M3,
    PA_READ_PROBE_SINK_WORDS,
    pa_cache_write,
    pa_cache_write_fp8,
    pa_copy_blocks,
    pa_compute_slots,
    pa_append_decode,
    pa_append_decode_fp8,
    pa_decode,
    pa_decode_fp8,
    pa_decode_noalloc,
    PA_NOALLOC_SCRATCH_BYTES,
    pa_decode_partition_size,
    pa_decode_workspace_size,
    pa_last_error,
    pa_prefill,
    pa_prefill_fp8,
    pa_read_probe,
    pa_version,
)
