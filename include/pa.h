/*
 * pa.h -- C ABI of libpa.so: paged KV-cache decode for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources cited below by short key:
 *   P1  "大模型部署中的PagedAttention：KV Cache显存管理突破" (PagedAttention in LLM
 *       deployment: a breakthrough in KV-cache memory management),
 *       blog.csdn.net/qq_22409661/article/details/146144360
 *   P2  "大模型推理优化：KV Cache与PagedAttention技术详解" (LLM inference
 *       optimisation: KV cache and PagedAttention explained),
 *       intelliparadigm.com/article/weixin_32678995/2221576
 *   P3  "LLM 推理中的 PageAttention 实现原理：虚拟内存管理在 KV Cache 中的创新应用"
 *       (How PageAttention works in LLM inference), www.dpshk.com/news/3461484/
 *
 * Conventions shared by every entry point
 *   - Every array pointer is a DEVICE pointer to memory the caller owns; the
 *     library never allocates, frees or keeps device memory (the one
 *     exception: the static per-GPU scratch array of pa_decode_noalloc, part
 *     of the loaded code), never synchronises the host, and launches only on
 *     the caller's `stream` (NULL = the null stream).  Calls return as soon
 *     as the work is queued.
 *   - Arrays are dense, row-major, with the shapes given per argument.
 *   - Storage types: PA_F32 (IEEE binary32), PA_F16 (IEEE binary16),
 *     PA_BF16 (bfloat16).  Arithmetic is float32 throughout.
 *   - KV pool layout: key_cache and value_cache are each
 *     [num_blocks][num_kv_heads][block_size][head_dim]: one physical block
 *     holds block_size consecutive tokens of a sequence (P1 §1, P3 §1), one
 *     (block, kv head) tile is block_size * head_dim contiguous elements.
 *   - Token t of sequence s lives in physical block
 *     block_tables[s][t / block_size] at offset t % block_size (P3 §3, the
 *     block table's lookup of a token index).  Indices are 0-based.
 *   - Query head h reads kv head h / (num_heads / num_kv_heads).
 *   - Errors: a non-OK status means nothing was launched; pa_last_error()
 *     then describes the failure.  Values that live in device memory
 *     (context_lens, block ids, slots, positions) cannot be checked by the
 *     host; the kernels check them instead, as stated per entry point, and
 *     never read or write outside the arrays described here.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* PA_FP8_E4M3 is a K/V pool type only (pa_cache_write_fp8, pa_decode_fp8, and
 * the dtype argument of the sizing functions for those pools): OCP FP8 E4M3
 * codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7F and 0xFF
 * are NaN; largest finite 448), one float32 scale per pool, value = code *
 * scale. */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, H % Hkv != 0, ... */
  PA_ERR_UNSUPPORTED = 2,        /* valid but not built: head_dim, block_size, dtype */
  PA_ERR_WORKSPACE_TOO_SMALL = 3,
  PA_ERR_HIP = 4,                /* the HIP runtime refused the launch */
  PA_ERR_NO_BLOCKS = 5,          /* block manager: not enough free blocks */
  PA_ERR_UNKNOWN_REQUEST = 6,    /* block manager: no table for this request id */
  PA_ERR_STATE = 7               /* block manager: operation invalid in this state */
} pa_status_t;

/*
 * pa_compute_slots -- resolve tokens to pool slots (P3 §3: logical block =
 * t / B, offset = t % B, physical block = table[logical]; P3 §2: the block
 * table maps each token to its block).
 *
 *   slot_mapping   out  int64 [num_tokens]; slot = phys * block_size + offset,
 *                       or -1 for a token that has no valid slot.
 *   block_tables   in   int32 [num_seqs][max_blocks_per_seq]
 *   context_lens   in   int32 [num_seqs] or NULL (needed when positions is NULL)
 *   seq_ids        in   int32 [num_tokens] or NULL: token i belongs to
 *                       sequence seq_ids[i] (NULL: to sequence i)
 *   positions      in   int32 [num_tokens] or NULL: the token's 0-based
 *                       position; NULL = the newest token of its sequence,
 *                       context_lens[seq] - 1 (P2 §2.1: the new token's K/V
 *                       are appended before attention reads the cache).
 *
 * A token gets -1 when its sequence id is outside [0, num_seqs), its position
 * is negative, its logical block is >= max_blocks_per_seq, or its table entry
 * is outside [0, num_blocks).
 */
pa_status_t pa_compute_slots(int64_t *slot_mapping, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *context_lens,
                             const int32_t *seq_ids, const int32_t *positions,
                             int32_t num_tokens, int32_t num_seqs, int32_t block_size,
                             int32_t num_blocks, hipStream_t stream);

/*
 * pa_cache_write -- write new tokens' K and V into their pool slots (P2 §2.1
 * step 3, the current token's K/V join the cache; the slot is the one P3 §3
 * assigns).  A bit-exact copy:
 *   key_cache[slot / B][h][slot % B][:] = key[i][h][:]   (same for value)
 *
 *   key, value           in     [num_tokens][num_kv_heads][head_dim]
 *   key_cache, value_cache in/out [num_blocks][num_kv_heads][block_size][head_dim]
 *   slot_mapping         in     int64 [num_tokens]
 *
 * Tokens whose slot is outside [0, num_blocks * block_size) (e.g. -1 padding)
 * are skipped.  Two tokens with the same slot in one call race: the result
 * is one of the two rows, unspecified which.
 * Supported: head_dim % (16 / element bytes) == 0, any block_size >= 1.
 */
pa_status_t pa_cache_write(const void *key, const void *value, void *key_cache,
                           void *value_cache, const int64_t *slot_mapping,
                           int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, pa_dtype_t dtype,
                           hipStream_t stream);

/*
 * pa_decode_partition_size -- the split-context partition length pa_decode
 * uses for these sizes.  `partition_size` > 0 is validated and returned as
 * is; 0 asks the library to choose.  Returns -1 for invalid sizes (see
 * pa_last_error).  A return value >= max_context_len means one partition per
 * sequence (no merge pass, no workspace).
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_context_len, int32_t partition_size,
                                 pa_dtype_t dtype);

/*
 * pa_decode_workspace_size -- bytes of device workspace pa_decode needs for
 * these sizes (0 when one partition covers max_context_len).  Returns
 * (size_t)-1 for invalid sizes.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size,
                                int32_t max_context_len, int32_t partition_size,
                                pa_dtype_t dtype);

/*
 * pa_decode -- PagedAttention decode (P1 §1 first formula; P2 §2.1 steps
 * 4-5; P3 §2, attention gathers each token's K/V through
 * block_tables[sequence]):
 *
 *   out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s
 *
 * over tokens t < context_lens[s] of sequence s, K_s/V_s gathered from the
 * pools through the sequence's block table.  Long contexts are split into
 * partitions of `partition_size` tokens whose (max, sum, unnormalised
 * output) states are merged exactly by a log-sum-exp pass.  (P1 §1's second
 * formula, a sum of per-block softmaxes, is not this quantity and is not
 * computed.)
 *
 *   out            out  [num_seqs][num_heads][head_dim], storage type dtype
 *   q              in   [num_seqs][num_heads][head_dim]
 *   key_cache, value_cache in [num_blocks][num_kv_heads][block_size][head_dim]
 *   block_tables   in   int32 [num_seqs][max_blocks_per_seq]; entries past a
 *                       sequence's ceil(ctx / block_size) blocks are never read
 *   context_lens   in   int32 [num_seqs], tokens to attend (the newest
 *                       token included)
 *   max_context_len     host-side upper bound on context_lens
 *   scale               score scale, normally 1/sqrt(head_dim) (P1 §1)
 *   partition_size      tokens per split-context partition, 0 = choose;
 *                       must be a multiple of block_size and of 16
 *   workspace           device memory of >= pa_decode_workspace_size(...)
 *                       bytes, 256-byte aligned, or NULL when that size is
 *                       0; the caller's, its contents on entry do not
 *                       matter.  Memory the GPU cannot reach (pageable host
 *                       memory) is refused with PA_ERR_INVALID_ARGUMENT;
 *                       pinned host memory is accepted.
 *
 * A sequence with context_lens[s] == 0 gets zeros.  A sequence whose
 * context_lens value is negative or above max_context_len or
 * max_blocks_per_seq * block_size, or whose used table entries fall outside
 * [0, num_blocks), gets NaN in every output element instead of a result.
 * Supported: head_dim in {64, 128}; block_size in {16, 32, 64};
 * num_heads % num_kv_heads == 0.  fp16/bf16 with num_heads / num_kv_heads
 * >= 2 run on the matrix cores (one work item per kv head and tile of up to
 * 16 of its query heads); fp32, and one query head per kv head, run on the
 * vector units (one work item per query head).
 */
pa_status_t pa_decode(void *out, const void *q, const void *key_cache, const void *value_cache,
                      const int32_t *block_tables, const int32_t *context_lens,
                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                      int32_t partition_size, void *workspace, size_t workspace_bytes,
                      pa_dtype_t dtype, hipStream_t stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes no workspace: the split-context partials go to
 * a static device array of PA_NOALLOC_SCRATCH_BYTES (16 MiB) that each GPU the
 * library runs on holds until the process ends.  The call itself allocates
 * nothing (no hipMalloc, no hipFree); the first call on a device looks up
 * that device's copy of the array.
 *
 * Arguments and results as for pa_decode (fp32/fp16/bf16 pools), minus
 * workspace and workspace_bytes.  A split that needs more than
 * PA_NOALLOC_SCRATCH_BYTES (pa_decode_workspace_size) is refused with
 * PA_ERR_WORKSPACE_TOO_SMALL before anything is launched; 16 MiB holds, e.g.,
 * 8 sequences x 32 heads x 64 partitions of a 128-dim head (8.5 MB).
 * Every call on one GPU shares that GPU's array and leaves its partials
 * there (nothing in it needs clearing: every partial read is written first
 * by the same call); calls that overlap on one GPU (different streams, or
 * host threads) race on it and must be serialised by the caller.
 */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)
pa_status_t pa_decode_noalloc(void *out, const void *q, const void *key_cache,
                              const void *value_cache, const int32_t *block_tables,
                              const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t max_context_len, float scale, int32_t partition_size,
                              pa_dtype_t dtype, hipStream_t stream);

/*
 * pa_append_decode -- one decode step in one launch: for every sequence s
 * with context_lens[s] >= 1, token t = context_lens[s] - 1 is the newest
 * one.  Its K/V rows (key[s], value[s]) are written to its slot
 * block_tables[s][t / block_size] * block_size + t % block_size (the cache
 * write of P2 §2.1 and P3 §3, with the slot resolved as pa_compute_slots
 * does), and out[s] is pa_decode's result over tokens 0..t, the newest
 * token's K/V taken from key/value.  Outputs and the pools afterwards are
 * bit-identical to pa_compute_slots + pa_cache_write + pa_decode on the same
 * inputs.
 *
 *   key, value     in   [num_seqs][num_kv_heads][head_dim], storage type
 *                       dtype, 16-byte aligned: the newest token's rows
 *   key_cache, value_cache  in/out  the pools, as for pa_decode
 *   every other argument as for pa_decode.
 *
 * Sequences with context_lens[s] == 0 write nothing and get zeros.  Outputs
 * are poisoned (NaN) exactly as pa_decode's.  The newest token's rows are
 * written whenever its context length is one pa_decode accepts and its own
 * block id lies inside the pool (a bad id elsewhere in the table poisons the
 * output but does not stop the write, as with pa_cache_write).  The slot of the
 * newest token must not be shared with another sequence's context (copy a
 * shared last block first, pa_copy_blocks).  dtype PA_F32, PA_F16 or PA_BF16
 * (E4M3 pools: pa_append_decode_fp8).
 */
pa_status_t pa_append_decode(void *out, const void *q, const void *key, const void *value,
                             void *key_cache, void *value_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t max_context_len, float scale, int32_t partition_size,
                             void *workspace, size_t workspace_bytes, pa_dtype_t dtype,
                             hipStream_t stream);

/*
 * pa_append_decode_fp8 -- pa_append_decode over E4M3 pools: the newest
 * token's rows (key/value, [num_seqs][num_kv_heads][head_dim] in q_dtype,
 * PA_F16 or PA_BF16) are quantised with the pool scales exactly as
 * pa_cache_write_fp8 does and stored in their slot, and out[s] is
 * pa_decode_fp8's result over tokens 0..t with the newest token's stored
 * codes.  Pools afterwards are bit-identical to pa_compute_slots +
 * pa_cache_write_fp8 on the same inputs; other rules as pa_append_decode and
 * pa_decode_fp8.
 */
pa_status_t pa_append_decode_fp8(void *out, const void *q, const void *key,
                                 const void *value, void *key_cache, void *value_cache,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                 float scale, float k_scale, float v_scale,
                                 int32_t partition_size, void *workspace,
                                 size_t workspace_bytes, pa_dtype_t q_dtype,
                                 hipStream_t stream);

/*
 * pa_prefill -- paged attention for many query tokens per sequence (a prompt,
 * or the new part of a prompt whose prefix is already cached), on the matrix
 * cores.  The pages give the per-token step (P2 §2.1: the token's K/V join
 * the cache, then its query attends over every cached K/V) and say that a
 * cached shared prefix spares its prefill work (P3 §3); this is that step
 * for every prompt token:
 *
 *   out[i][h] = softmax(scale * q[i][h] . K_s[0..p]^T) V_s[0..p]
 *
 * where row i is the j-th query row of sequence s (query_start[s] <= i <
 * query_start[s+1], j = i - query_start[s]), qlen = query_start[s+1] -
 * query_start[s], and p = context_lens[s] - qlen + j: the queries are the
 * last qlen tokens of the context, whose K/V the caller has already written
 * (pa_cache_write), and each attends causally to the tokens up to its own.
 *
 *   out            out  [num_tokens][num_heads][head_dim], dtype
 *   q              in   [num_tokens][num_heads][head_dim], dtype
 *   key_cache, value_cache, block_tables, num_blocks, max_blocks_per_seq:
 *                       as for pa_decode
 *   context_lens   in   int32 [num_seqs]: tokens in the cache, queries included
 *   query_start    in   int32 [num_seqs + 1], non-decreasing, query_start[0]
 *                       = 0, query_start[num_seqs] = num_tokens
 *   max_query_len       host-side upper bound on every qlen (<= max_context_len)
 *
 * Rows of a sequence whose device values are inconsistent (context length
 * negative or above max_context_len or max_blocks_per_seq * block_size; qlen
 * negative, above its context or above max_query_len; query_start outside
 * [0, num_tokens]), or whose used table entries fall outside [0, num_blocks),
 * get NaN; other sequences are unaffected.  Supported: fp16, bf16; head_dim
 * 64 or 128; block_size 16, 32 or 64; num_heads % num_kv_heads == 0.
 */
pa_status_t pa_prefill(void *out, const void *q, const void *key_cache, const void *value_cache,
                       const int32_t *block_tables, const int32_t *context_lens,
                       const int32_t *query_start, int32_t num_seqs, int32_t num_tokens,
                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                       int32_t max_query_len, int32_t max_context_len, float scale,
                       pa_dtype_t dtype, hipStream_t stream);

/*
 * pa_prefill_fp8 -- pa_prefill over E4M3 pools (the lower-precision cache of
 * P1 §4-§5 and P2 §5, in the reading pa_cache_write_fp8 documents): a
 * prompt's query rows attend causally to a context whose K/V are stored as
 * codes, value = decode(code) * k_scale (K) or * v_scale (V), e.g. a cached
 * prefix written by pa_cache_write_fp8 (P3 §3).  Row j of sequence s at
 * position p = context_lens[s] - qlen + j gets
 *   out = softmax(scale * q . k_t, t = 0..p) . v_t
 * over those values, computed in float32.
 *   key_cache, value_cache  in  uint8 E4M3 codes [num_blocks][num_kv_heads][block_size][head_dim]
 *   k_scale, v_scale        in  the pools' scales (finite, > 0)
 *   dtype                   q's and out's type: PA_F16 or PA_BF16
 *   every other argument as for pa_prefill.
 * Errors as for pa_prefill; PA_ERR_INVALID_ARGUMENT for a scale that is not
 * finite and positive.  Device-resident values poison only their rows, as
 * for pa_prefill.
 */
pa_status_t pa_prefill_fp8(void *out, const void *q, const void *key_cache,
                           const void *value_cache, const int32_t *block_tables,
                           const int32_t *context_lens, const int32_t *query_start,
                           int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                           int32_t max_context_len, float scale, float k_scale, float v_scale,
                           pa_dtype_t dtype, hipStream_t stream);

/*
 * pa_cache_write_fp8 -- pa_cache_write into E4M3 pools.  The pages advise
 * keeping the cache in a lower precision to save memory (P1 §4 keeps blocks
 * in bfloat16; P1 §5 and P2 §5 quantise and compress the cache); the reading
 * taken here is 8-bit E4M3 codes with one float32 scale per pool.  Each element
 * x of a new row (storage type src_dtype, widened exactly to float32) is
 * stored as the E4M3 code nearest to x / scale (IEEE float32 division), ties
 * to the even code, magnitudes above 448 saturated to 448, NaN as 0x7F:
 *   key_cache[slot / B][h][slot % B][d] = code(key[i][h][d] / k_scale)
 * (the same for value with v_scale).  Bit-exact by definition.
 *
 *   key, value             in     [num_tokens][num_kv_heads][head_dim], src_dtype
 *   key_cache, value_cache in/out uint8 [num_blocks][num_kv_heads][block_size][head_dim]
 *   slot_mapping           in     int64 [num_tokens]; out-of-range slots are skipped
 *   k_scale, v_scale             finite and > 0
 * Supported: head_dim a multiple of 16; src_dtype PA_F32, PA_F16 or PA_BF16.
 */
pa_status_t pa_cache_write_fp8(const void *key, const void *value, void *key_cache,
                               void *value_cache, const int64_t *slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, pa_dtype_t src_dtype,
                               float k_scale, float v_scale, hipStream_t stream);

/*
 * pa_decode_fp8 -- pa_decode over E4M3 pools: attention over the stored
 * values code * k_scale (keys) and code * v_scale (values); q and out are
 * fp16 or bf16 (q_dtype), arithmetic is float32.  Every other argument,
 * the partition and workspace rules (size them with dtype PA_FP8_E4M3) and
 * the handling of invalid device values are those of pa_decode.  With
 * num_heads / num_kv_heads >= 2 it runs on the matrix cores (the codes
 * widened exactly to q's type), otherwise on the vector units.
 */
pa_status_t pa_decode_fp8(void *out, const void *q, const void *key_cache,
                          const void *value_cache, const int32_t *block_tables,
                          const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t max_context_len, float scale, float k_scale, float v_scale,
                          int32_t partition_size, void *workspace, size_t workspace_bytes,
                          pa_dtype_t q_dtype, hipStream_t stream);

/*
 * pa_copy_blocks -- copy whole physical blocks from one pair of pools to
 * another, for copy on write inside a pool (P3 §4: a beam fork shares block
 * references; a request that writes into a shared block needs its own copy,
 * see pa_blocks.h) and for swapping a preempted request's blocks out to host
 * memory and back in (P3 §3, §5: blocks of low-priority requests move to CPU
 * memory and return when GPU blocks are free).  A bit-exact copy:
 *
 *   dst_k[dst] = src_k[src],  dst_v[dst] = src_v[src]   for each pair
 *
 *   dst_k, dst_v     out  pools of dst_num_blocks blocks of block_bytes each
 *   src_k, src_v     in   pools of src_num_blocks blocks of block_bytes each
 *                         (dst_v and src_v may both be NULL: one pool only)
 *   block_pairs      in   int32 [num_pairs][2] = (src block, dst block), in
 *                         device or pinned host memory
 *   block_bytes           bytes of one physical block (num_kv_heads *
 *                         block_size * head_dim * element bytes for the
 *                         layouts of pa_decode); a multiple of 16
 *
 * Every pool pointer is device memory, or pinned host memory from
 * hipHostMalloc (mapped into the device address space: the kernel then
 * reads or writes across the host link); the library asks the HIP runtime
 * for each pointer's device view and returns PA_ERR_INVALID_ARGUMENT for
 * memory a kernel cannot reach.  Pools must be 16-byte aligned.  A
 * pair whose src or dst is outside its pool is skipped.  Pairs are copied in
 * no particular order: a block that is the dst of one pair and the src of
 * another in the same call gives an unspecified result.
 */
pa_status_t pa_copy_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                           const int32_t *block_pairs, int32_t num_pairs, int64_t block_bytes,
                           int32_t dst_num_blocks, int32_t src_num_blocks, hipStream_t stream);

/*
 * pa_read_probe -- the achievable HBM read rate for a tiled pattern, to set
 * beside the nominal peak (the decode kernels read 4 KB (block, kv head)
 * tiles of K and V in table order, i.e. scattered).  Reads num_tiles tiles of
 * tile_bytes from buf in the order given (order[i] = index of the i-th tile
 * read; NULL reads them in index order; entries outside [0, num_tiles) are
 * clamped), 16-byte non-temporal loads, 1 KB per wave load, and writes per
 * work-group the XOR of every 32-bit word it read to sink (so the XOR of all
 * sink words is the XOR of the buffer when order is a permutation).
 *
 *   buf       in   device, >= tile_bytes * num_tiles bytes, 16-byte aligned
 *   order     in   device int32 [num_tiles] or NULL
 *   sink      out  device, PA_READ_PROBE_SINK_WORDS uint32 words, overwritten
 *
 * tile_bytes must be a positive multiple of 1024.  The caller times the call.
 */
#define PA_READ_PROBE_SINK_WORDS 2048
pa_status_t pa_read_probe(const void *buf, int64_t tile_bytes, int64_t num_tiles,
                          const int32_t *order, uint32_t *sink, hipStream_t stream);

/* Text of the last non-OK status returned on the calling thread. */
const char *pa_last_error(void);

/* Library version string. */
const char *pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
