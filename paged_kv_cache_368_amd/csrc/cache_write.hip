// Paged cache write (reshape-and-cache) and slot resolution for gfx950.
//
// cache write: each new token's K and V rows are copied bit for bit into
// their pool slot (P2 §2.1 step 3: the current token's K/V join the cache),
//   key_cache[slot / B][h][slot % B][:] = key[i][h][:].
// A thread moves U 16-byte pieces of K rows and the matching pieces of V
// rows (a work-group covers U x 256 consecutive pieces, so loads and stores
// are full 16-byte accesses over whole rows), issuing all its loads before
// the slot lookups and stores; the rows are read once and the slots written
// once, so both go non-temporal.  U = 4 for large writes (a prompt's rows:
// 3% faster than one piece per thread), U = 1 for a decode step's few rows,
// where more work-groups with shorter chains finish sooner (2.8 against
// 6.1 us for 64 tokens of 40 heads).
//
// slot resolution (P3 §3): logical block = t / B, offset = t % B,
// slot = block_tables[seq][logical] * B + offset.
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kCwThreads = 256;
constexpr long long kCwLarge = 1 << 20;   // pieces from which U = 4 is used

template <int U>
__global__ __launch_bounds__(kCwThreads) void cache_write_kernel(
    const u32x4 *__restrict__ key, const u32x4 *__restrict__ value, u32x4 *__restrict__ key_cache,
    u32x4 *__restrict__ value_cache, const int64_t *__restrict__ slot_mapping, int num_tokens,
    int num_kv_heads, int row_units, int block_size, long long pool_slots) {
  const long long per_token = (long long)num_kv_heads * row_units;
  const long long total = per_token * num_tokens;
  const long long base = (long long)blockIdx.x * (kCwThreads * U) + threadIdx.x;
  u32x4 kv[U], vv[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const long long u = base + j * kCwThreads;
    if (u < total) {
      kv[j] = __builtin_nontemporal_load(key + u);
      vv[j] = __builtin_nontemporal_load(value + u);
    }
  }
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const long long u = base + j * kCwThreads;
    if (u >= total) break;
    const long long i = u / per_token;
    const int rem = (int)(u - i * per_token);           // h * row_units + c
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= pool_slots) continue;
    const long long blk = slot / block_size;
    const int off = (int)(slot - blk * block_size);
    const int h = rem / row_units;
    const int c = rem - h * row_units;
    const long long dst = ((blk * num_kv_heads + h) * block_size + off) * row_units + c;
    __builtin_nontemporal_store(kv[j], key_cache + dst);
    __builtin_nontemporal_store(vv[j], value_cache + dst);
  }
}

__global__ __launch_bounds__(256) void compute_slots_kernel(
    int64_t *__restrict__ slot_mapping, const int32_t *__restrict__ block_tables,
    int max_blocks_per_seq, const int32_t *__restrict__ context_lens,
    const int32_t *__restrict__ seq_ids, const int32_t *__restrict__ positions, int num_tokens,
    int num_seqs, int block_size, int num_blocks) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= num_tokens) return;
  int64_t slot = -1;
  const int s = seq_ids ? seq_ids[i] : i;
  if (s >= 0 && s < num_seqs) {
    const int pos = positions ? positions[i] : context_lens[s] - 1;
    if (pos >= 0) {
      const int logical = pos / block_size;
      const int offset = pos - logical * block_size;
      if (logical < max_blocks_per_seq) {
        const int phys = block_tables[(size_t)s * max_blocks_per_seq + logical];
        if (phys >= 0 && phys < num_blocks) slot = (int64_t)phys * block_size + offset;
      }
    }
  }
  slot_mapping[i] = slot;
}

// Cache write into E4M3 pools: one thread converts 16 elements of a K row
// (and of the matching V row) and stores their 16 codes with one 16-byte
// store.  ST: the source rows' storage type.
template <int ST>
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(
    const char *__restrict__ key, const char *__restrict__ value, uint8_t *__restrict__ key_cache,
    uint8_t *__restrict__ value_cache, const int64_t *__restrict__ slot_mapping, int num_tokens,
    int num_kv_heads, int head_dim, int block_size, long long pool_slots, float k_scale,
    float v_scale) {
  constexpr int ES = Storage<ST>::kBytes;
  constexpr int SW = 16 * ES / 16;                          // 16-byte source words per piece
  const int pieces = head_dim / 16;
  const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long per_token = (long long)num_kv_heads * pieces;
  if (u >= per_token * num_tokens) return;
  const int i = (int)(u / per_token);
  const int rem = (int)(u - (long long)i * per_token);
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= pool_slots) return;
  const long long blk = slot / block_size;
  const int off = (int)(slot - blk * block_size);
  const int h = rem / pieces;
  const int c = rem - h * pieces;
  const long long src = (((long long)i * num_kv_heads + h) * head_dim + c * 16) * ES;
  const long long dst = ((blk * num_kv_heads + h) * block_size + off) * head_dim + c * 16;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const char *in = (which == 0 ? key : value) + src;
    const float scale = which == 0 ? k_scale : v_scale;
    u32x4 w[SW];
#pragma unroll
    for (int j = 0; j < SW; ++j) w[j] = reinterpret_cast<const u32x4 *>(in)[j];
    *reinterpret_cast<u32x4 *>((which == 0 ? key_cache : value_cache) + dst) =
        e4m3_codes16<ST>(w, scale);
  }
}

}  // namespace

hipError_t launch_cache_write_fp8(const void *key, const void *value, void *key_cache,
                                  void *value_cache, const int64_t *slot_mapping, int num_tokens,
                                  int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  int src_dt, float k_scale, float v_scale, hipStream_t stream) {
  const long long total = (long long)num_tokens * num_kv_heads * (head_dim / 16);
  if (total <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  const long long slots = (long long)num_blocks * block_size;
  const char *k = static_cast<const char *>(key), *v = static_cast<const char *>(value);
  uint8_t *kc = static_cast<uint8_t *>(key_cache), *vc = static_cast<uint8_t *>(value_cache);
  switch (src_dt) {
    case kF32:
      hipLaunchKernelGGL(cache_write_fp8_kernel<kF32>, dim3(grid), dim3(256), 0, stream, k, v, kc,
                         vc, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, slots,
                         k_scale, v_scale);
      break;
    case kF16:
      hipLaunchKernelGGL(cache_write_fp8_kernel<kF16>, dim3(grid), dim3(256), 0, stream, k, v, kc,
                         vc, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, slots,
                         k_scale, v_scale);
      break;
    case kBF16:
      hipLaunchKernelGGL(cache_write_fp8_kernel<kBF16>, dim3(grid), dim3(256), 0, stream, k, v,
                         kc, vc, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size,
                         slots, k_scale, v_scale);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cache_write(const void *key, const void *value, void *key_cache,
                              void *value_cache, const int64_t *slot_mapping, int num_tokens,
                              int num_kv_heads, int row_bytes, int block_size, int num_blocks,
                              hipStream_t stream) {
  const int row_units = row_bytes / 16;
  const long long total = (long long)num_tokens * num_kv_heads * row_units;
  if (total <= 0) return hipSuccess;
  const bool large = total >= kCwLarge;
  const long long per_wg = kCwThreads * (large ? 4 : 1);
  const unsigned grid = (unsigned)((total + per_wg - 1) / per_wg);
  hipLaunchKernelGGL(large ? cache_write_kernel<4> : cache_write_kernel<1>, dim3(grid),
                     dim3(kCwThreads), 0, stream,
                     reinterpret_cast<const u32x4 *>(key), reinterpret_cast<const u32x4 *>(value),
                     reinterpret_cast<u32x4 *>(key_cache), reinterpret_cast<u32x4 *>(value_cache),
                     slot_mapping, num_tokens, num_kv_heads, row_units, block_size,
                     (long long)num_blocks * block_size);
  return hipGetLastError();
}

hipError_t launch_compute_slots(int64_t *slot_mapping, const int32_t *block_tables,
                                int max_blocks_per_seq, const int32_t *context_lens,
                                const int32_t *seq_ids, const int32_t *positions,
                                int num_tokens, int num_seqs, int block_size, int num_blocks,
                                hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((num_tokens + 255) / 256);
  hipLaunchKernelGGL(compute_slots_kernel, dim3(grid), dim3(256), 0, stream, slot_mapping,
                     block_tables, max_blocks_per_seq, context_lens, seq_ids, positions,
                     num_tokens, num_seqs, block_size, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
