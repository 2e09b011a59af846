// Whole-block copies between pools for gfx950 (include/pa.h pa_copy_blocks):
// copy on write inside a device pool (P3 §4, a beam fork shares blocks that
// a writer must then copy) and swapping blocks out to pinned host memory and
// back in (P3 §3, §5).
//
// One wave moves one 1 KB piece of a block, of the K pool and (when given)
// the same piece of the V pool: each lane issues its 16-byte loads before its
// stores.  The pieces of one pair run on one XCD, next to each other in its
// dispatch order (xcd_major): with random block ids, consecutive pieces of a
// block on the round-robin order's eight XCDs cost ~8% (measured on MI355X:
// 2048 random pairs of 160 KB bf16 blocks, K and V, 5.85 against 5.40 TB/s
// read + write; 16 KB work-groups of 4 waves, as before, 5.1 TB/s).
// Device-pool traffic is marked non-temporal (read once, written once).  A
// pair with an id outside its pool is skipped.
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kCopyThreads = 64;
constexpr long long kCopyPiece = kCopyThreads * 16;     // 1 KB

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    char *dst_k, char *dst_v, const char *src_k, const char *src_v, const int32_t *pairs,
    long long block_bytes, int pieces, long long items, int dst_num_blocks, int src_num_blocks) {
  const long long item = xcd_major(blockIdx.x, items);
  const int pair = (int)(item / pieces);
  const int piece = (int)(item - (long long)pair * pieces);
  const int src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  if (src < 0 || src >= src_num_blocks || dst < 0 || dst >= dst_num_blocks) return;
  const long long off = piece * kCopyPiece + threadIdx.x * 16;
  if (off >= block_bytes) return;
  const long long s = (long long)src * block_bytes + off;
  const long long d = (long long)dst * block_bytes + off;
  const u32x4 k = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src_k + s));
  u32x4 v = {0u, 0u, 0u, 0u};
  if (dst_v) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src_v + s));
  __builtin_nontemporal_store(k, reinterpret_cast<u32x4 *>(dst_k + d));
  if (dst_v) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst_v + d));
}

}  // namespace

hipError_t launch_copy_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                              const int32_t *pairs, int num_pairs, long long block_bytes,
                              int dst_num_blocks, int src_num_blocks, hipStream_t stream) {
  const long long pieces = (block_bytes + kCopyPiece - 1) / kCopyPiece;
  const long long n = (long long)num_pairs * pieces;
  if (n <= 0) return hipSuccess;
  if (n > 0x7fffffffLL || pieces > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n), dim3(kCopyThreads), 0, stream,
                     static_cast<char *>(dst_k), static_cast<char *>(dst_v),
                     static_cast<const char *>(src_k), static_cast<const char *>(src_v), pairs,
                     block_bytes, (int)pieces, n, dst_num_blocks, src_num_blocks);
  return hipGetLastError();
}

}  // namespace pa
