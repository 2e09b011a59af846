// Whole-block copies between pools for gfx950 (include/pa.h pa_copy_blocks):
// copy on write inside a device pool (P3 §4, a beam fork shares blocks that
// a writer must then copy) and swapping blocks out to pinned host memory and
// back in (P3 §3, §5).
//
// One work-group of 256 threads moves one 16 KB piece of one block of one
// pool: each thread issues its four 16-byte loads before any store, so a
// work-group keeps 16 KB in flight.  Device-pool traffic is marked
// non-temporal (read once, written once).  A pair with an id outside its
// pool is skipped.
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr long long kCopyPiece = (long long)kCopyThreads * kCopyUnroll * 16;   // 16 KB

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    char *dst_k, char *dst_v, const char *src_k, const char *src_v, const int32_t *pairs,
    long long block_bytes, int pieces, int pools, int dst_num_blocks, int src_num_blocks) {
  const int per_pair = pieces * pools;
  const int pair = blockIdx.x / per_pair;
  const int rem = blockIdx.x - pair * per_pair;
  const int pool = rem / pieces;
  const int piece = rem - pool * pieces;
  const int src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  if (src < 0 || src >= src_num_blocks || dst < 0 || dst >= dst_num_blocks) return;
  const char *s = (pool == 0 ? src_k : src_v) + (long long)src * block_bytes;
  char *d = (pool == 0 ? dst_k : dst_v) + (long long)dst * block_bytes;
  const long long base = piece * kCopyPiece + threadIdx.x * 16;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const long long off = base + (long long)u * kCopyThreads * 16;
    if (off < block_bytes)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(s + off));
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const long long off = base + (long long)u * kCopyThreads * 16;
    if (off < block_bytes) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4 *>(d + off));
  }
}

}  // namespace

hipError_t launch_copy_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                              const int32_t *pairs, int num_pairs, long long block_bytes,
                              int dst_num_blocks, int src_num_blocks, hipStream_t stream) {
  const int pools = dst_v ? 2 : 1;
  const long long pieces = (block_bytes + kCopyPiece - 1) / kCopyPiece;
  const long long n = (long long)num_pairs * pieces * pools;
  if (n <= 0) return hipSuccess;
  if (n > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n), dim3(kCopyThreads), 0, stream,
                     static_cast<char *>(dst_k), static_cast<char *>(dst_v),
                     static_cast<const char *>(src_k), static_cast<const char *>(src_v), pairs,
                     block_bytes, (int)pieces, pools, dst_num_blocks, src_num_blocks);
  return hipGetLastError();
}

}  // namespace pa
