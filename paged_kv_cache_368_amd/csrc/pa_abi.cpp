// C ABI of libpa.so (declared in include/pa.h): argument validation, the
// choice of split-context partition length, workspace sizing and kernel
// dispatch.  Allocates nothing, never synchronises, launches on the caller's
// stream.
#include "pa.h"

#include <math.h>

#include <atomic>
#include <mutex>
#include <string>

#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

pa_status_t fail(pa_status_t st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// The address a kernel uses for a pool that is device memory or pinned host
// memory (hipHostMalloc, mapped into the device address space).  Returns
// nullptr for anything else (pageable host memory, unknown pointers), so no
// kernel is ever handed an address it cannot reach.
const void *device_view(const void *p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();                  // clear the runtime's record of the query
    return nullptr;
  }
  switch (at.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
    case hipMemoryTypeUnified:
      return p;
    case hipMemoryTypeHost:
      return at.devicePointer;
    default:
      return nullptr;
  }
}

// The automatic partition length.  Measured on MI355X: longer partitions are
// faster (fewer work-group prologues, no merge pass when one partition covers
// the context), so one partition per context up to 4096 tokens, 2048-token
// partitions beyond that, shortened only while the grid would leave CUs
// without a work-group (256 CUs).
constexpr long long kMinWorkgroups = 256;

struct Sizes {
  int partition;
  int num_partitions;
  size_t ws_o_bytes;
  size_t ws_bytes;
};

pa_status_t check_shape(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t max_context_len,
                        pa_dtype_t dtype) {
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
  if (num_heads <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_heads and num_kv_heads must be > 0");
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_heads must be a multiple of num_kv_heads");
  if (max_context_len < 0) return fail(PA_ERR_INVALID_ARGUMENT, "max_context_len must be >= 0");
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16 && dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "dtype must be PA_F32, PA_F16, PA_BF16 or PA_FP8_E4M3");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (block_size != 16 && block_size != 32 && block_size != 64)
    return fail(PA_ERR_UNSUPPORTED, "block_size must be 16, 32 or 64");
  return PA_OK;
}

pa_status_t plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                 int32_t block_size, int32_t max_context_len, int32_t partition_size,
                 pa_dtype_t dtype, Sizes *out) {
  pa_status_t st = check_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                               max_context_len, dtype);
  if (st != PA_OK) return st;
  int P = partition_size;
  if (P < 0) return fail(PA_ERR_INVALID_ARGUMENT, "partition_size must be >= 0");
  if (P > 0) {
    if (P % block_size != 0 || P % pa::kChunk != 0)
      return fail(PA_ERR_INVALID_ARGUMENT,
                  "partition_size must be a multiple of block_size and of 16");
    if (P > pa::kMaxPartition)
      return fail(PA_ERR_UNSUPPORTED, "partition_size above 4096 tokens is not supported");
  } else {
    // Work items are (sequence, query head) on the vector kernel and
    // (sequence, kv head) on the matrix-core grouped-query kernel.
    const bool gqa = pa::gqa_supported(dtype, head_dim, num_heads, num_kv_heads);
    const long long tiles = ceil_div(num_heads / num_kv_heads, pa::kGqaTile);
    const long long items = (long long)num_seqs * (gqa ? num_kv_heads * tiles : num_heads);
    // The matrix-core kernel does the same per-token work over E4M3 pools
    // for half the bytes: it was measured fastest with two work-groups per CU.
    const long long min_wg = gqa && dtype == PA_FP8_E4M3 ? 2 * kMinWorkgroups : kMinWorkgroups;
    P = max_context_len > pa::kMaxPartition ? pa::kMaxPartition / 2 : pa::kMaxPartition;
    while (P > 256 && items * ceil_div(max_context_len, P) < min_wg) P /= 2;
  }
  const long long np = max_context_len > 0 ? ceil_div(max_context_len, P) : 1;
  if ((long long)num_seqs * num_heads * np > 0x7fffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "too many (sequence, head, partition) work items");
  out->partition = P;
  out->num_partitions = (int)np;
  out->ws_o_bytes = 0;
  out->ws_bytes = 0;
  if (np > 1) {
    const size_t parts = (size_t)num_seqs * num_heads * (size_t)np;
    out->ws_o_bytes = (parts * head_dim * sizeof(float) + 255) & ~(size_t)255;
    out->ws_bytes = out->ws_o_bytes + parts * 2 * sizeof(float);
  }
  return PA_OK;
}

}  // namespace

pa_status_t pa::set_error(pa_status_t st, const char *msg) { return fail(st, msg); }

extern "C" {

const char *pa_last_error(void) { return g_last_error.c_str(); }

const char *pa_version(void) { return "pa 0.1.0 gfx950"; }

pa_status_t pa_compute_slots(int64_t *slot_mapping, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *context_lens,
                             const int32_t *seq_ids, const int32_t *positions,
                             int32_t num_tokens, int32_t num_seqs, int32_t block_size,
                             int32_t num_blocks, hipStream_t stream) {
  if (num_tokens < 0 || num_seqs < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens and num_seqs must be >= 0");
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping || !block_tables)
    return fail(PA_ERR_INVALID_ARGUMENT, "slot_mapping and block_tables must not be NULL");
  if (!positions && !context_lens)
    return fail(PA_ERR_INVALID_ARGUMENT, "positions or context_lens must be given");
  if (max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "max_blocks_per_seq, block_size and num_blocks must be > 0");
  hipError_t e = pa::launch_compute_slots(slot_mapping, block_tables, max_blocks_per_seq,
                                          context_lens, seq_ids, positions, num_tokens,
                                          num_seqs, block_size, num_blocks, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return PA_OK;
}

pa_status_t pa_cache_write(const void *key, const void *value, void *key_cache,
                           void *value_cache, const int64_t *slot_mapping,
                           int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, pa_dtype_t dtype,
                           hipStream_t stream) {
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "dtype must be PA_F32, PA_F16 or PA_BF16");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0");
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "num_kv_heads, head_dim, block_size and num_blocks must be > 0");
  const int row_bytes = head_dim * pa::elem_bytes(dtype);
  if (row_bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "head_dim * element bytes must be a multiple of 16");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARGUMENT, "pointer arguments must not be NULL");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "key, value and the pools must be 16-byte aligned");
  hipError_t e = pa::launch_cache_write(key, value, key_cache, value_cache, slot_mapping,
                                        num_tokens, num_kv_heads, row_bytes, block_size,
                                        num_blocks, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return PA_OK;
}

pa_status_t pa_copy_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                           const int32_t *block_pairs, int32_t num_pairs, int64_t block_bytes,
                           int32_t dst_num_blocks, int32_t src_num_blocks, hipStream_t stream) {
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_pairs must be >= 0");
  if (block_bytes <= 0 || block_bytes % 16 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "block_bytes must be a positive multiple of 16");
  if (dst_num_blocks <= 0 || src_num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "dst_num_blocks and src_num_blocks must be > 0");
  if (num_pairs == 0) return PA_OK;
  if (!dst_k || !src_k || !block_pairs)
    return fail(PA_ERR_INVALID_ARGUMENT, "dst_k, src_k and block_pairs must not be NULL");
  if (!dst_v != !src_v)
    return fail(PA_ERR_INVALID_ARGUMENT, "dst_v and src_v must both be given or both be NULL");
  if (!aligned16(dst_k) || !aligned16(src_k) || (dst_v && (!aligned16(dst_v) || !aligned16(src_v))))
    return fail(PA_ERR_INVALID_ARGUMENT, "pools must be 16-byte aligned");
  const void *views[4] = {dst_k, dst_v, src_k, src_v};
  for (int i = 0; i < 4; ++i) {
    if (!views[i]) continue;
    views[i] = device_view(views[i]);
    if (!views[i])
      return fail(PA_ERR_INVALID_ARGUMENT,
                  "every pool must be device memory or pinned (hipHostMalloc) host memory");
  }
  const int32_t *pairs = static_cast<const int32_t *>(device_view(block_pairs));
  if (!pairs)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "block_pairs must be device memory or pinned (hipHostMalloc) host memory");
  hipError_t e = pa::launch_copy_blocks(const_cast<void *>(views[0]), const_cast<void *>(views[1]),
                                        views[2], views[3], pairs, num_pairs, block_bytes,
                                        dst_num_blocks, src_num_blocks, stream);
  if (e == hipErrorInvalidValue)
    return fail(PA_ERR_UNSUPPORTED, "too many pairs for one launch");
  if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return PA_OK;
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_context_len, int32_t partition_size,
                                 pa_dtype_t dtype) {
  Sizes z;
  if (plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
           partition_size, dtype, &z) != PA_OK)
    return -1;
  return z.partition;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size,
                                int32_t max_context_len, int32_t partition_size,
                                pa_dtype_t dtype) {
  Sizes z;
  if (plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
           partition_size, dtype, &z) != PA_OK)
    return (size_t)-1;
  return z.ws_bytes;
}

}  // extern "C"

namespace {

// pa_decode and pa_decode_fp8: q/out of type q_dt, pools of type kv_dt
// (q_dt, or PA_FP8_E4M3 with its two pool scales).
pa_status_t decode_impl(void *out, const void *q, const void *key_cache, const void *value_cache,
                        const int32_t *block_tables, const int32_t *context_lens,
                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                        int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                        float k_scale, float v_scale, int32_t partition_size, void *workspace,
                        size_t workspace_bytes, pa_dtype_t q_dt, pa_dtype_t kv_dt,
                        hipStream_t stream, const void *new_k = nullptr,
                        const void *new_v = nullptr, bool workspace_is_device = false) {
  Sizes z;
  pa_status_t st = plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_context_len, partition_size, kv_dt, &z);
  if (st != PA_OK) return st;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks and max_blocks_per_seq must be > 0");
  if ((long long)max_context_len > (long long)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "max_context_len exceeds max_blocks_per_seq * block_size");
  if (!isfinite(scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (!isfinite(k_scale) || !isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return fail(PA_ERR_INVALID_ARGUMENT, "k_scale and v_scale must be finite and > 0");
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !key_cache || !value_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARGUMENT, "pointer arguments must not be NULL");
  if (!aligned16(out) || !aligned16(q) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "out, q and the pools must be 16-byte aligned");
  if ((new_k == nullptr) != (new_v == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "key and value must both be given");
  if (new_k && (!aligned16(new_k) || !aligned16(new_v)))
    return fail(PA_ERR_INVALID_ARGUMENT, "key and value must be 16-byte aligned");
  if (z.ws_bytes > 0) {
    if (!workspace || workspace_bytes < z.ws_bytes)
      return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                  "workspace smaller than pa_decode_workspace_size() = " +
                      std::to_string(z.ws_bytes) + " bytes");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(PA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    // The kernels write the partials there: refuse memory the GPU cannot
    // reach (pageable host memory) instead of handing it to them.
    if (!workspace_is_device) workspace = const_cast<void *>(device_view(workspace));
    if (!workspace)
      return fail(PA_ERR_INVALID_ARGUMENT,
                  "workspace must be device memory or pinned (hipHostMalloc) host memory");
  }

  pa::DecodeArgs a;
  a.out = out;
  a.ws_o = static_cast<float *>(workspace);
  a.ws_ml = z.ws_bytes ? reinterpret_cast<float *>(static_cast<char *>(workspace) + z.ws_o_bytes)
                       : nullptr;
  a.q = q;
  a.k_cache = key_cache;
  a.v_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.log2_block = ilog2(block_size);
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.scale_log2 = scale * 1.4426950408889634f * k_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.partition_size = z.partition;
  a.num_partitions = z.num_partitions;
  a.new_k = new_k;
  a.new_v = new_v;
  a.k_store = const_cast<void *>(key_cache);
  a.v_store = const_cast<void *>(value_cache);

  hipError_t e = pa::gqa_supported(kv_dt, head_dim, num_heads, num_kv_heads)
                     ? pa::launch_decode_gqa(a, q_dt, kv_dt, stream)
                     : pa::launch_decode_mha(a, q_dt, kv_dt, stream);
  if (e == hipSuccess && z.num_partitions > 1) e = pa::launch_merge(a, q_dt, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t pa_decode(void *out, const void *q, const void *key_cache, const void *value_cache,
                      const int32_t *block_tables, const int32_t *context_lens,
                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                      int32_t partition_size, void *workspace, size_t workspace_bytes,
                      pa_dtype_t dtype, hipStream_t stream) {
  if (dtype == PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "E4M3 pools are decoded by pa_decode_fp8");
  return decode_impl(out, q, key_cache, value_cache, block_tables, context_lens, num_seqs,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, 1.f, 1.f, partition_size,
                     workspace, workspace_bytes, dtype, dtype, stream);
}

pa_status_t pa_append_decode(void *out, const void *q, const void *key, const void *value,
                             void *key_cache, void *value_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t max_context_len, float scale, int32_t partition_size,
                             void *workspace, size_t workspace_bytes, pa_dtype_t dtype,
                             hipStream_t stream) {
  if (dtype == PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "E4M3 pools are appended by pa_append_decode_fp8");
  if (num_seqs > 0 && (!key || !value))
    return fail(PA_ERR_INVALID_ARGUMENT, "pointer arguments must not be NULL");
  return decode_impl(out, q, key_cache, value_cache, block_tables, context_lens, num_seqs,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, 1.f, 1.f, partition_size,
                     workspace, workspace_bytes, dtype, dtype, stream, key, value);
}

pa_status_t pa_append_decode_fp8(void *out, const void *q, const void *key,
                                 const void *value, void *key_cache, void *value_cache,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                 float scale, float k_scale, float v_scale,
                                 int32_t partition_size, void *workspace,
                                 size_t workspace_bytes, pa_dtype_t q_dtype,
                                 hipStream_t stream) {
  if (q_dtype != PA_F16 && q_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_append_decode_fp8 takes fp16 or bf16 queries and rows");
  if (num_seqs > 0 && (!key || !value))
    return fail(PA_ERR_INVALID_ARGUMENT, "pointer arguments must not be NULL");
  return decode_impl(out, q, key_cache, value_cache, block_tables, context_lens, num_seqs,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, k_scale, v_scale,
                     partition_size, workspace, workspace_bytes, q_dtype, PA_FP8_E4M3, stream,
                     key, value);
}

pa_status_t pa_decode_fp8(void *out, const void *q, const void *key_cache,
                          const void *value_cache, const int32_t *block_tables,
                          const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t max_context_len, float scale, float k_scale, float v_scale,
                          int32_t partition_size, void *workspace, size_t workspace_bytes,
                          pa_dtype_t q_dtype, hipStream_t stream) {
  if (q_dtype != PA_F16 && q_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_fp8 takes fp16 or bf16 queries");
  return decode_impl(out, q, key_cache, value_cache, block_tables, context_lens, num_seqs,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, k_scale, v_scale,
                     partition_size, workspace, workspace_bytes, q_dtype, PA_FP8_E4M3, stream);
}

}  // extern "C"

// pa_decode_noalloc's workspace: one static device array per GPU, held until
// the process ends.  Host code never uses the array's own name as an address
// (on the host it is only a stand-in); it uses the per-device address that
// hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch address on the device that `stream` belongs to (the current
// device for the null stream).  The first call on a device makes that device
// current, looks the address up and restores the caller's device.
pa_status_t scratch_for(hipStream_t stream, void **ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(PA_ERR_HIP, std::string("device of the stream: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "device index above 63");
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = -1;
      e = hipGetDevice(&cur);
      if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
      if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur >= 0 && cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
      }
      if (e != hipSuccess || !p)
        return fail(PA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                    hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t pa_decode_noalloc(void *out, const void *q, const void *key_cache,
                              const void *value_cache, const int32_t *block_tables,
                              const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t max_context_len, float scale, int32_t partition_size,
                              pa_dtype_t dtype, hipStream_t stream) {
  if (dtype == PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_noalloc takes PA_F32, PA_F16 or PA_BF16 pools");
  Sizes z;
  pa_status_t st = plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_context_len, partition_size, dtype, &z);
  if (st != PA_OK) return st;
  if (z.ws_bytes > PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                "this split needs " + std::to_string(z.ws_bytes) +
                    " bytes of workspace, above the static scratch of " +
                    std::to_string((size_t)PA_NOALLOC_SCRATCH_BYTES) +
                    " bytes: use pa_decode with a workspace, or longer partitions");
  void *ws = nullptr;
  if (z.ws_bytes > 0 && num_seqs > 0) {
    st = scratch_for(stream, &ws);
    if (st != PA_OK) return st;
  }
  return decode_impl(out, q, key_cache, value_cache, block_tables, context_lens, num_seqs,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, scale, 1.f, 1.f, partition_size, ws,
                     ws ? (size_t)PA_NOALLOC_SCRATCH_BYTES : 0, dtype, dtype, stream, nullptr,
                     nullptr, /*workspace_is_device=*/true);
}

}  // extern "C"

namespace {

// pa_prefill and pa_prefill_fp8: q/out of type dtype, pools of type kv_dt
// (dtype, or PA_FP8_E4M3 with its two pool scales).
pa_status_t prefill_impl(void *out, const void *q, const void *key_cache, const void *value_cache,
                         const int32_t *block_tables, const int32_t *context_lens,
                         const int32_t *query_start, int32_t num_seqs, int32_t num_tokens,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_query_len, int32_t max_context_len, float scale,
                         float k_scale, float v_scale, pa_dtype_t dtype, pa_dtype_t kv_dt,
                         hipStream_t stream) {
  pa_status_t st = check_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                               max_context_len, dtype);
  if (st != PA_OK) return st;
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, kv_dt == PA_FP8_E4M3 ? "pa_prefill_fp8 takes fp16 or bf16 queries"
                                                          : "pa_prefill takes fp16 or bf16");
  if (kv_dt == PA_FP8_E4M3 && !(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) &&
                                v_scale > 0.f))
    return fail(PA_ERR_INVALID_ARGUMENT, "k_scale and v_scale must be finite and > 0");
  if (num_tokens < 0 || max_query_len < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens and max_query_len must be >= 0");
  if (max_query_len > max_context_len)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_query_len exceeds max_context_len");
  if (num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks and max_blocks_per_seq must be > 0");
  if ((long long)max_context_len > (long long)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "max_context_len exceeds max_blocks_per_seq * block_size");
  if (!isfinite(scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !key_cache || !value_cache || !block_tables || !context_lens || !query_start)
    return fail(PA_ERR_INVALID_ARGUMENT, "pointer arguments must not be NULL");
  if (!aligned16(out) || !aligned16(q) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "out, q and the pools must be 16-byte aligned");
  const long long tiles = ceil_div(max_query_len, pa::prefill_rows_per_tile());
  if ((long long)num_seqs * num_heads * tiles > 0x7fffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "too many (sequence, head, query tile) work items");
  pa::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = key_cache;
  a.v_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.log2_block = ilog2(block_size);
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.max_context_len = max_context_len;
  a.num_tiles = (int)tiles;
  a.scale_log2 = scale * (kv_dt == PA_FP8_E4M3 ? k_scale : 1.f) * 1.4426950408889634f;
  a.v_scale = kv_dt == PA_FP8_E4M3 ? v_scale : 1.f;
  hipError_t e = pa::launch_prefill(a, dtype, kv_dt, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t pa_prefill(void *out, const void *q, const void *key_cache, const void *value_cache,
                       const int32_t *block_tables, const int32_t *context_lens,
                       const int32_t *query_start, int32_t num_seqs, int32_t num_tokens,
                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                       int32_t max_query_len, int32_t max_context_len, float scale,
                       pa_dtype_t dtype, hipStream_t stream) {
  return prefill_impl(out, q, key_cache, value_cache, block_tables, context_lens, query_start,
                      num_seqs, num_tokens, num_heads, num_kv_heads, head_dim, block_size,
                      num_blocks, max_blocks_per_seq, max_query_len, max_context_len, scale, 1.f,
                      1.f, dtype, dtype, stream);
}

pa_status_t pa_prefill_fp8(void *out, const void *q, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *context_lens, const int32_t *query_start,
                           int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                           int32_t max_context_len, float scale, float k_scale, float v_scale,
                           pa_dtype_t dtype, hipStream_t stream) {
  return prefill_impl(out, q, key_cache, value_cache, block_tables, context_lens, query_start,
                      num_seqs, num_tokens, num_heads, num_kv_heads, head_dim, block_size,
                      num_blocks, max_blocks_per_seq, max_query_len, max_context_len, scale,
                      k_scale, v_scale, dtype, PA_FP8_E4M3, stream);
}

pa_status_t pa_cache_write_fp8(const void *key, const void *value, void *key_cache,
                               void *value_cache, const int64_t *slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, pa_dtype_t src_dtype,
                               float k_scale, float v_scale, hipStream_t stream) {
  if (src_dtype != PA_F32 && src_dtype != PA_F16 && src_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "src_dtype must be PA_F32, PA_F16 or PA_BF16");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0");
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "num_kv_heads, head_dim, block_size and num_blocks must be > 0");
  if (head_dim % 16 != 0) return fail(PA_ERR_UNSUPPORTED, "head_dim must be a multiple of 16");
  if (!isfinite(k_scale) || !isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return fail(PA_ERR_INVALID_ARGUMENT, "k_scale and v_scale must be finite and > 0");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARGUMENT, "pointer arguments must not be NULL");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "key, value and the pools must be 16-byte aligned");
  hipError_t e = pa::launch_cache_write_fp8(key, value, key_cache, value_cache, slot_mapping,
                                            num_tokens, num_kv_heads, head_dim, block_size,
                                            num_blocks, src_dtype, k_scale, v_scale, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return PA_OK;
}

pa_status_t pa_read_probe(const void *buf, int64_t tile_bytes, int64_t num_tiles,
                          const int32_t *order, uint32_t *sink, hipStream_t stream) {
  if (tile_bytes <= 0 || tile_bytes % 1024 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "tile_bytes must be a positive multiple of 1024");
  if (num_tiles < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_tiles must be >= 0");
  if (num_tiles == 0) return PA_OK;
  if (!buf || !sink) return fail(PA_ERR_INVALID_ARGUMENT, "pointer arguments must not be NULL");
  if (!aligned16(buf)) return fail(PA_ERR_INVALID_ARGUMENT, "buf must be 16-byte aligned");
  const hipError_t e = pa::launch_read_probe(buf, tile_bytes, num_tiles, order, sink, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return PA_OK;
}

}  // extern "C"
