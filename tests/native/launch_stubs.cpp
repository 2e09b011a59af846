// Launch entry points for a CPU-only build of the library's host code (the
// C ABI's validation and dispatch, and the block manager) under the
// sanitizers: there are no kernels, so every launch reports that no device
// is present, as the real library does on a machine without a GPU.
#include "pa_internal.h"

namespace pa {

hipError_t launch_prefill(const PrefillArgs &, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_mha(const DecodeArgs &, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_merge(const DecodeArgs &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_gqa(const DecodeArgs &, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_cache_write(const void *, const void *, void *, void *, const int64_t *, int,
                              int, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_copy_blocks(void *, void *, const void *, const void *, const int32_t *, int,
                              long long, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_cache_write_fp8(const void *, const void *, void *, void *, const int64_t *,
                                  int, int, int, int, int, int, float, float, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_read_probe(const void *, long long, long long, const int32_t *, uint32_t *,
                             hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_compute_slots(int64_t *, const int32_t *, int, const int32_t *, const int32_t *,
                                const int32_t *, int, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace pa
