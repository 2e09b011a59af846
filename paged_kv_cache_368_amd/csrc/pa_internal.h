// Internal launch interface between the C ABI (pa_abi.cpp) and the kernels.
// Not installed; the public surface is include/pa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Record the thread's last error text (read back by pa_last_error) and
// return `st`.  Defined in pa_abi.cpp.
pa_status_t set_error(pa_status_t st, const char *msg);

// Storage types; kFP8 (OCP E4M3 codes with a per-pool scale) is a KV-pool type only.
enum Dt : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

inline int elem_bytes(int dt) { return dt == kF32 ? 4 : dt == kFP8 ? 1 : 2; }

// Longest partition one work-group handles: 256 chunks of 16 tokens.  Bounded
// by the per-wave block-id register (64 lanes x 4 waves) and by the LDS copy
// of the partition's table slice.
constexpr int kMaxPartition = 4096;
constexpr int kChunk = 16;            // tokens per inner-loop step of a wave
// Work-group shapes and pipeline depths, each measured against its
// neighbours on MI355X (more waves per decode work-group, or a third K/V
// buffer, was no faster and cost occupancy).
constexpr int kDecodeWaves = 4;       // waves per decode work-group
constexpr int kDecodeBuffers = 2;     // K/V chunk buffers in flight per wave
constexpr int kDecodeBuffersFp8 = 2;  // the same for 8-bit pools
constexpr int kGqaWaves = 4;          // waves per grouped-query work-group
constexpr int kGqaBuffers = 2;        // K/V chunk buffers per grouped-query wave
constexpr int kMaxPartBlocks = kMaxPartition / 16;

struct DecodeArgs {
  void *out;                 // [S][H][D] storage dtype
  float *ws_o;               // [S][H][NP][D] fp32, unnormalised partial outputs
  float *ws_ml;              // [S][H][NP][2] fp32, (max score in log2 units, sum)
  const void *q;             // [S][H][D]
  const void *k_cache;       // [NB][Hkv][B][D]
  const void *v_cache;
  const int32_t *block_tables;  // [S][MB]
  const int32_t *context_lens;  // [S]
  int num_seqs, num_heads, num_kv_heads, head_dim;
  int block_size, log2_block, num_blocks, max_blocks_per_seq, max_context_len;
  float scale_log2;          // scale * log2(e) (* the K pool scale for fp8 pools): base-2 scores
  float k_scale;             // the K pool scale for fp8 pools (1 otherwise)
  float v_scale;             // the V pool scale for fp8 pools (1 otherwise)
  int partition_size;        // P
  int num_partitions;        // NP = ceil(max_context_len / P), >= 1
  int parts_per_group;       // consecutive partitions per vector work-group (set by its launch)
  // Appending decode (null otherwise): token context_lens[s] - 1 of every
  // sequence is new; its K/V rows [S][Hkv][D] are attended from here and
  // written to the token's slot in the pools (k_store/v_store: the pools).
  const void *new_k;
  const void *new_v;
  void *k_store;
  void *v_store;
};

// kv_dt: the pools' storage type, equal to dt or kFP8 (dt fp16/bf16 only).
struct PrefillArgs {
  void *out;                 // [T][H][D]
  const void *q;             // [T][H][D]
  const void *k_cache;       // [NB][Hkv][B][D]
  const void *v_cache;
  const int32_t *block_tables;  // [S][MB]
  const int32_t *context_lens;  // [S]
  const int32_t *query_start;   // [S + 1]
  int num_seqs, num_tokens, num_heads, num_kv_heads, head_dim;
  int block_size, log2_block, num_blocks, max_blocks_per_seq;
  int max_query_len, max_context_len;
  int num_tiles;             // ceil(max_query_len / rows per tile)
  float scale_log2;          // score scale (times the K scale over E4M3 pools) x log2(e)
  float v_scale;             // E4M3 pools: the V scale, applied to the outputs
};

// Paged prefill on the matrix cores: fp16/bf16, head_dim 64 or 128; one
// work-group per tile of kPrefillRows query rows of one (sequence, head).
constexpr int kPrefillRows = 256;
inline int prefill_rows_per_tile() { return kPrefillRows; }
hipError_t launch_prefill(const PrefillArgs &a, int dt, int kv_dt, hipStream_t stream);

hipError_t launch_decode_mha(const DecodeArgs &a, int dt, int kv_dt, hipStream_t stream);
hipError_t launch_merge(const DecodeArgs &a, int dt, hipStream_t stream);

// Grouped-query decode on the matrix cores: fp16/bf16 queries over pools of
// the same type or of E4M3 codes (kv_dt), head_dim 64 or 128,
// num_heads / num_kv_heads >= 2.  One work item per (sequence, kv head,
// tile of up to kGqaTile query heads, partition) instead of per query head.
constexpr int kGqaTile = 16;
inline bool gqa_supported(int kv_dt, int head_dim, int num_heads, int num_kv_heads) {
  return (kv_dt == kF16 || kv_dt == kBF16 || kv_dt == kFP8) &&
         (head_dim == 64 || head_dim == 128) && num_heads / num_kv_heads >= 2;
}
hipError_t launch_decode_gqa(const DecodeArgs &a, int dt, int kv_dt, hipStream_t stream);

hipError_t launch_cache_write(const void *key, const void *value, void *key_cache,
                              void *value_cache, const int64_t *slot_mapping, int num_tokens,
                              int num_kv_heads, int row_bytes, int block_size, int num_blocks,
                              hipStream_t stream);

hipError_t launch_copy_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                              const int32_t *pairs, int num_pairs, long long block_bytes,
                              int dst_num_blocks, int src_num_blocks, hipStream_t stream);

// Cache write into E4M3 pools: rows of src_dt widened to float32, divided by
// the pool's scale and rounded to the nearest code (ties to even), saturated.
hipError_t launch_cache_write_fp8(const void *key, const void *value, void *key_cache,
                                  void *value_cache, const int64_t *slot_mapping, int num_tokens,
                                  int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  int src_dt, float k_scale, float v_scale, hipStream_t stream);

// Read-bandwidth probe (one uint32 of sink per work-group).
hipError_t launch_read_probe(const void *buf, long long tile_bytes, long long num_tiles,
                             const int32_t *order, uint32_t *sink, hipStream_t stream);

hipError_t launch_compute_slots(int64_t *slot_mapping, const int32_t *block_tables,
                                int max_blocks_per_seq, const int32_t *context_lens,
                                const int32_t *seq_ids, const int32_t *positions,
                                int num_tokens, int num_seqs, int block_size, int num_blocks,
                                hipStream_t stream);

}  // namespace pa
