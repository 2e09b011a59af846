/*
 * pa_blocks.h -- host-side KV block manager of libpa.so: the block pool and
 * per-request block tables whose output (block tables, slots) feeds
 * pa_cache_write and pa_decode (pa.h).
 *
 * Sources, cited by short key as in pa.h:
 *   P3 §3  the Rust paged KV-cache manager: a pool of fixed-size blocks with
 *          a FIFO free queue and a reference count per block; per-request
 *          block tables; all-or-nothing allocation for a prompt; append_slot
 *          for decoding; release of a request; prefix sharing by reference.
 *   P3 §4  beam search forks a request by copying its block references.
 *
 * Semantics (readings of points the listing leaves open or contradicts):
 *   - Reference counts live with the block: allocation sets 1, sharing adds
 *     1, release subtracts 1 and returns the block to the back of the free
 *     queue at 0.  Releasing or sharing a block whose count is 0 is an error
 *     (PA_ERR_STATE), never a saturation.
 *   - Token positions are 0-based: position p lives in logical block
 *     p / block_size at offset p % block_size; slot = phys * block_size +
 *     offset (the slot pa_cache_write takes).
 *   - Appending position p allocates logical block p / block_size when it is
 *     the first block past the table; a position further out is PA_ERR_STATE.
 *   - Appending into a block that another request also holds is copy on
 *     write: the request drops its reference, gets a fresh block, and the
 *     call reports (src, dst); the caller copies src into dst on the device
 *     (pa_copy_blocks) before writing the new token.
 *
 * Threading: every call on one manager is serialised by the manager's own
 * mutex; distinct managers are independent.  All memory is host memory owned
 * by the manager, released by pa_bm_destroy.  Errors: a non-OK status leaves
 * the manager unchanged (except where stated for pa_bm_append_slots) and
 * pa_last_error() describes it.
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A pool of num_blocks blocks of block_size tokens, all free, queued in id
 * order 0 .. num_blocks-1 (P3 §3 BlockPool::new). */
pa_status_t pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager **out);

/* Release the manager and everything it holds (NULL is ignored). */
void pa_bm_destroy(pa_block_manager *bm);

/* All-or-nothing allocation of ceil(num_tokens / block_size) blocks for a new
 * request (P3 §3 allocate_for_request).  PA_ERR_NO_BLOCKS when the free queue
 * is too short (nothing is taken); PA_ERR_STATE when request_id already has a
 * table.  *num_blocks_out (may be NULL) receives the block count. */
pa_status_t pa_bm_allocate(pa_block_manager *bm, uint64_t request_id, int32_t num_tokens,
                           int32_t *num_blocks_out);

/* Make room for the token at `position` of a request (P3 §3 append_slot).
 *   slot_out        its slot (phys * block_size + offset)
 *   new_block_out   the block allocated by this call, or -1
 *   copy_src_out, copy_dst_out  the copy-on-write pair, or -1, -1
 * Any out pointer may be NULL.  PA_ERR_NO_BLOCKS when a block is needed and
 * none is free (preemption is the caller's decision); PA_ERR_UNKNOWN_REQUEST;
 * PA_ERR_STATE for a position past the next block. */
pa_status_t pa_bm_append_slot(pa_block_manager *bm, uint64_t request_id, int32_t position,
                              int64_t *slot_out, int32_t *new_block_out, int32_t *copy_src_out,
                              int32_t *copy_dst_out);

/* pa_bm_append_slot over n (request, position) pairs in order, for one
 * decode step: slots[i] receives each slot, copy_pairs (int32 [n][2], may be
 * NULL) the copy-on-write pairs in the order they arose, *num_copies their
 * count.  Stops at the first failure: *num_done (may be NULL) is the number
 * of pairs applied, and those stay applied. */
pa_status_t pa_bm_append_slots(pa_block_manager *bm, const uint64_t *request_ids,
                               const int32_t *positions, int32_t n, int64_t *slots,
                               int32_t *copy_pairs, int32_t *num_copies, int32_t *num_done);

/* dst gets the first ceil(shared_len / block_size) blocks of src, each with
 * one more reference (P3 §3 share_prefix_blocks).  PA_ERR_STATE when dst
 * already has a table or src holds fewer blocks. */
pa_status_t pa_bm_share_prefix(pa_block_manager *bm, uint64_t src_request_id,
                               uint64_t dst_request_id, int32_t shared_len);

/* Beam fork (P3 §4): dst shares every block of src. */
pa_status_t pa_bm_fork(pa_block_manager *bm, uint64_t src_request_id, uint64_t dst_request_id);

/* Release every block reference of a request and forget it (P3 §3
 * free_request).  PA_ERR_UNKNOWN_REQUEST for an unknown id. */
pa_status_t pa_bm_free_request(pa_block_manager *bm, uint64_t request_id);

/* Counters: free blocks, allocated blocks (total - free), live requests.
 * Any out pointer may be NULL.  P3 §3's usage ratio is allocated / total. */
pa_status_t pa_bm_stats(const pa_block_manager *bm, int32_t *num_free, int32_t *num_allocated,
                        int32_t *num_requests);

/* Reference count of one block, or -1 for an id outside the pool. */
int32_t pa_bm_ref_count(const pa_block_manager *bm, int32_t block_id);

/* Copy a request's block table (logical order) into blocks[0 .. capacity);
 * *len receives its full length.  PA_ERR_INVALID_ARGUMENT when capacity is
 * smaller than the length (nothing is copied). */
pa_status_t pa_bm_table(const pa_block_manager *bm, uint64_t request_id, int32_t *blocks,
                        int32_t capacity, int32_t *len);

/* Copy the free queue, front first, into ids[0 .. capacity); *len receives
 * its full length (same capacity rule as pa_bm_table). */
pa_status_t pa_bm_free_ids(const pa_block_manager *bm, int32_t *ids, int32_t capacity,
                           int32_t *len);

/* Fill a HOST array tables[num_seqs][max_blocks_per_seq] with the tables of
 * the given requests, padded with -1: the block_tables argument of pa_decode
 * (the caller copies it to the device).  PA_ERR_UNKNOWN_REQUEST for an
 * unknown id; PA_ERR_INVALID_ARGUMENT when a table is longer than
 * max_blocks_per_seq.  Nothing is written on error. */
pa_status_t pa_bm_fill_tables(const pa_block_manager *bm, const uint64_t *request_ids,
                              int32_t num_seqs, int32_t max_blocks_per_seq, int32_t *tables);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */
