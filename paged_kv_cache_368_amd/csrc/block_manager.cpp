// Host-side KV block manager (include/pa_blocks.h): the block pool with its
// FIFO free queue and reference counts, and the per-request block tables of
// P3 §3, with prefix sharing and the beam fork of P3 §4.  Plain C++ behind
// one mutex per manager; no GPU work.
#include "pa_blocks.h"

#include <deque>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_queue;               // front = next to allocate
  std::vector<int32_t> ref;                     // references per block
  std::unordered_map<uint64_t, std::vector<int32_t>> tables;
  mutable std::mutex mu;
};

namespace {

using Table = std::vector<int32_t>;

pa_status_t fail(pa_status_t st, const std::string &msg) { return pa::set_error(st, msg.c_str()); }

int64_t blocks_for(int64_t tokens, int32_t block_size) {
  return (tokens + block_size - 1) / block_size;
}

// Pool primitives (caller holds the lock).
int32_t take_front(pa_block_manager *bm) {
  const int32_t b = bm->free_queue.front();
  bm->free_queue.pop_front();
  bm->ref[b] = 1;
  return b;
}

void release(pa_block_manager *bm, int32_t b) {
  if (--bm->ref[b] == 0) bm->free_queue.push_back(b);
}

std::string rid_text(uint64_t rid) { return std::to_string((unsigned long long)rid); }

// One append (caller holds the lock); on error nothing has changed.
pa_status_t append_locked(pa_block_manager *bm, uint64_t rid, int32_t position, int64_t *slot,
                          int32_t *new_block, int32_t *copy_src, int32_t *copy_dst) {
  auto it = bm->tables.find(rid);
  if (it == bm->tables.end())
    return fail(PA_ERR_UNKNOWN_REQUEST, "request " + rid_text(rid) + " not found");
  if (position < 0) return fail(PA_ERR_INVALID_ARGUMENT, "position must be >= 0");
  Table &t = it->second;
  const int64_t logical = position / bm->block_size;
  const int32_t offset = position % bm->block_size;
  if (logical > (int64_t)t.size())
    return fail(PA_ERR_STATE, "position " + std::to_string(position) +
                                  " skips past the end of the request's table");
  int32_t nb = -1, csrc = -1, cdst = -1;
  if (logical == (int64_t)t.size()) {
    if (bm->free_queue.empty())
      return fail(PA_ERR_NO_BLOCKS, "preemption required: no free blocks");
    nb = take_front(bm);
    t.push_back(nb);
  } else if (bm->ref[t[logical]] > 1) {
    // Copy on write: the shared block keeps its other holders.
    if (bm->free_queue.empty())
      return fail(PA_ERR_NO_BLOCKS, "preemption required: no free block for copy on write");
    nb = take_front(bm);
    csrc = t[logical];
    cdst = nb;
    release(bm, csrc);
    t[logical] = nb;
  }
  if (slot) *slot = (int64_t)t[logical] * bm->block_size + offset;
  if (new_block) *new_block = nb;
  if (copy_src) *copy_src = csrc;
  if (copy_dst) *copy_dst = cdst;
  return PA_OK;
}

pa_status_t share_locked(pa_block_manager *bm, uint64_t src, uint64_t dst, int64_t shared_len) {
  auto it = bm->tables.find(src);
  if (it == bm->tables.end())
    return fail(PA_ERR_UNKNOWN_REQUEST, "source request " + rid_text(src) + " not found");
  if (shared_len < 0) return fail(PA_ERR_INVALID_ARGUMENT, "shared_len must be >= 0");
  if (bm->tables.count(dst))
    return fail(PA_ERR_STATE, "request " + rid_text(dst) + " already has a table");
  const int64_t n = blocks_for(shared_len, bm->block_size);
  const Table &s = it->second;
  if ((int64_t)s.size() < n)
    return fail(PA_ERR_STATE, "source has fewer blocks than the shared length needs");
  Table t(s.begin(), s.begin() + n);
  for (int32_t b : t) ++bm->ref[b];
  bm->tables.emplace(dst, std::move(t));
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager **out) {
  if (!out) return fail(PA_ERR_INVALID_ARGUMENT, "out must not be NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks and block_size must be > 0");
  pa_block_manager *bm = new (std::nothrow) pa_block_manager;
  if (!bm) return fail(PA_ERR_INVALID_ARGUMENT, "out of host memory");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  for (int32_t b = 0; b < num_blocks; ++b) bm->free_queue.push_back(b);
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

pa_status_t pa_bm_allocate(pa_block_manager *bm, uint64_t request_id, int32_t num_tokens,
                           int32_t *num_blocks_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARGUMENT, "manager must not be NULL");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0");
  std::lock_guard<std::mutex> g(bm->mu);
  if (bm->tables.count(request_id))
    return fail(PA_ERR_STATE, "request " + rid_text(request_id) + " already has a table");
  const int64_t need = blocks_for(num_tokens, bm->block_size);
  if ((int64_t)bm->free_queue.size() < need)
    return fail(PA_ERR_NO_BLOCKS, "insufficient blocks: need " + std::to_string(need) +
                                      ", available " + std::to_string(bm->free_queue.size()));
  Table t;
  t.reserve(need);
  for (int64_t i = 0; i < need; ++i) t.push_back(take_front(bm));
  bm->tables.emplace(request_id, std::move(t));
  if (num_blocks_out) *num_blocks_out = (int32_t)need;
  return PA_OK;
}

pa_status_t pa_bm_append_slot(pa_block_manager *bm, uint64_t request_id, int32_t position,
                              int64_t *slot_out, int32_t *new_block_out, int32_t *copy_src_out,
                              int32_t *copy_dst_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARGUMENT, "manager must not be NULL");
  std::lock_guard<std::mutex> g(bm->mu);
  return append_locked(bm, request_id, position, slot_out, new_block_out, copy_src_out,
                       copy_dst_out);
}

pa_status_t pa_bm_append_slots(pa_block_manager *bm, const uint64_t *request_ids,
                               const int32_t *positions, int32_t n, int64_t *slots,
                               int32_t *copy_pairs, int32_t *num_copies, int32_t *num_done) {
  if (num_done) *num_done = 0;
  if (num_copies) *num_copies = 0;
  if (!bm) return fail(PA_ERR_INVALID_ARGUMENT, "manager must not be NULL");
  if (n < 0) return fail(PA_ERR_INVALID_ARGUMENT, "n must be >= 0");
  if (n > 0 && (!request_ids || !positions || !slots))
    return fail(PA_ERR_INVALID_ARGUMENT, "request_ids, positions and slots must not be NULL");
  std::lock_guard<std::mutex> g(bm->mu);
  int32_t copies = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src = -1, dst = -1;
    const pa_status_t st =
        append_locked(bm, request_ids[i], positions[i], &slots[i], nullptr, &src, &dst);
    if (st != PA_OK) return st;
    if (src >= 0) {
      if (copy_pairs) {
        copy_pairs[2 * copies] = src;
        copy_pairs[2 * copies + 1] = dst;
      }
      ++copies;
      if (num_copies) *num_copies = copies;
    }
    if (num_done) *num_done = i + 1;
  }
  return PA_OK;
}

pa_status_t pa_bm_share_prefix(pa_block_manager *bm, uint64_t src_request_id,
                               uint64_t dst_request_id, int32_t shared_len) {
  if (!bm) return fail(PA_ERR_INVALID_ARGUMENT, "manager must not be NULL");
  std::lock_guard<std::mutex> g(bm->mu);
  return share_locked(bm, src_request_id, dst_request_id, shared_len);
}

pa_status_t pa_bm_fork(pa_block_manager *bm, uint64_t src_request_id, uint64_t dst_request_id) {
  if (!bm) return fail(PA_ERR_INVALID_ARGUMENT, "manager must not be NULL");
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->tables.find(src_request_id);
  if (it == bm->tables.end())
    return fail(PA_ERR_UNKNOWN_REQUEST, "source request " + rid_text(src_request_id) + " not found");
  return share_locked(bm, src_request_id, dst_request_id,
                      (int64_t)it->second.size() * bm->block_size);
}

pa_status_t pa_bm_free_request(pa_block_manager *bm, uint64_t request_id) {
  if (!bm) return fail(PA_ERR_INVALID_ARGUMENT, "manager must not be NULL");
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->tables.find(request_id);
  if (it == bm->tables.end())
    return fail(PA_ERR_UNKNOWN_REQUEST, "request " + rid_text(request_id) + " not found");
  Table t = std::move(it->second);
  bm->tables.erase(it);
  for (int32_t b : t) release(bm, b);
  return PA_OK;
}

pa_status_t pa_bm_stats(const pa_block_manager *bm, int32_t *num_free, int32_t *num_allocated,
                        int32_t *num_requests) {
  if (!bm) return fail(PA_ERR_INVALID_ARGUMENT, "manager must not be NULL");
  std::lock_guard<std::mutex> g(bm->mu);
  const int32_t nf = (int32_t)bm->free_queue.size();
  if (num_free) *num_free = nf;
  if (num_allocated) *num_allocated = bm->num_blocks - nf;
  if (num_requests) *num_requests = (int32_t)bm->tables.size();
  return PA_OK;
}

int32_t pa_bm_ref_count(const pa_block_manager *bm, int32_t block_id) {
  if (!bm || block_id < 0 || block_id >= bm->num_blocks) return -1;
  std::lock_guard<std::mutex> g(bm->mu);
  return bm->ref[block_id];
}

pa_status_t pa_bm_table(const pa_block_manager *bm, uint64_t request_id, int32_t *blocks,
                        int32_t capacity, int32_t *len) {
  if (!bm || !len) return fail(PA_ERR_INVALID_ARGUMENT, "manager and len must not be NULL");
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->tables.find(request_id);
  if (it == bm->tables.end())
    return fail(PA_ERR_UNKNOWN_REQUEST, "request " + rid_text(request_id) + " not found");
  const Table &t = it->second;
  *len = (int32_t)t.size();
  if ((int64_t)t.size() > capacity || (t.size() && !blocks))
    return fail(PA_ERR_INVALID_ARGUMENT, "capacity smaller than the table");
  for (size_t i = 0; i < t.size(); ++i) blocks[i] = t[i];
  return PA_OK;
}

pa_status_t pa_bm_free_ids(const pa_block_manager *bm, int32_t *ids, int32_t capacity,
                           int32_t *len) {
  if (!bm || !len) return fail(PA_ERR_INVALID_ARGUMENT, "manager and len must not be NULL");
  std::lock_guard<std::mutex> g(bm->mu);
  *len = (int32_t)bm->free_queue.size();
  if ((int64_t)bm->free_queue.size() > capacity || (bm->free_queue.size() && !ids))
    return fail(PA_ERR_INVALID_ARGUMENT, "capacity smaller than the free queue");
  int32_t i = 0;
  for (int32_t b : bm->free_queue) ids[i++] = b;
  return PA_OK;
}

pa_status_t pa_bm_fill_tables(const pa_block_manager *bm, const uint64_t *request_ids,
                              int32_t num_seqs, int32_t max_blocks_per_seq, int32_t *tables) {
  if (!bm) return fail(PA_ERR_INVALID_ARGUMENT, "manager must not be NULL");
  if (num_seqs < 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 and max_blocks_per_seq > 0");
  if (num_seqs > 0 && (!request_ids || !tables))
    return fail(PA_ERR_INVALID_ARGUMENT, "request_ids and tables must not be NULL");
  std::lock_guard<std::mutex> g(bm->mu);
  for (int32_t s = 0; s < num_seqs; ++s) {
    auto it = bm->tables.find(request_ids[s]);
    if (it == bm->tables.end())
      return fail(PA_ERR_UNKNOWN_REQUEST, "request " + rid_text(request_ids[s]) + " not found");
    if ((int64_t)it->second.size() > max_blocks_per_seq)
      return fail(PA_ERR_INVALID_ARGUMENT, "request " + rid_text(request_ids[s]) +
                                               " holds more than max_blocks_per_seq blocks");
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    const Table &t = bm->tables.find(request_ids[s])->second;
    int32_t *row = tables + (size_t)s * max_blocks_per_seq;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < (int32_t)t.size() ? t[j] : -1;
  }
  return PA_OK;
}

}  // extern "C"
