// Multi-threaded stress of one host block manager (include/pa_blocks.h),
// built with the sanitizers on the CPU.  Every thread drives its own requests
// through allocate, append (with copy on write after forks), prefix sharing
// from one system prompt all threads share, beam forks, table and free-queue
// reads, and frees, while the others do the same on the same manager.  At the
// end every request is freed and the pool must be whole again: every block
// free exactly once, every reference count zero.
//
//   bm_threads [threads] [iterations]       exit status 0 = invariants held
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <thread>
#include <vector>

#include "pa_blocks.h"

namespace {

constexpr int32_t kBlocks = 2048;
constexpr int32_t kBlockSize = 16;
constexpr uint64_t kSystem = 1ull << 40;     // the shared system prompt's request id
constexpr int32_t kSystemTokens = 100;

struct Req {
  uint64_t id;
  int32_t len;
};

int worker(pa_block_manager *bm, int t, int iters) {
  std::mt19937_64 rng(1000 + t);
  std::vector<Req> live;
  uint64_t next = (uint64_t)(t + 1) << 32;
  int32_t table[512], free_ids[kBlocks];
  int32_t len = 0;
  int errors = 0;
  for (int i = 0; i < iters; ++i) {
    const int op = (int)(rng() % 100);
    if (op < 20 || live.empty()) {                       // new request
      const uint64_t id = next++;
      if (rng() % 3 == 0) {
        if (pa_bm_share_prefix(bm, kSystem, id, kSystemTokens) == PA_OK)
          live.push_back({id, kSystemTokens});
      } else {
        const int32_t n = 1 + (int32_t)(rng() % 300);
        if (pa_bm_allocate(bm, id, n, nullptr) == PA_OK) live.push_back({id, n});
      }
    } else if (op < 70) {                                 // decode-step appends
      Req &r = live[rng() % live.size()];
      int64_t slot;
      int32_t nb, cs, cd;
      const pa_status_t st = pa_bm_append_slot(bm, r.id, r.len, &slot, &nb, &cs, &cd);
      if (st == PA_OK) {
        if (slot < 0 || slot >= (int64_t)kBlocks * kBlockSize) ++errors;
        ++r.len;
      } else if (st != PA_ERR_NO_BLOCKS) {
        ++errors;
      }
    } else if (op < 78) {                                 // beam fork
      Req src = live[rng() % live.size()];
      const uint64_t id = next++;
      if (pa_bm_fork(bm, src.id, id) == PA_OK) live.push_back({id, src.len});
      else ++errors;
    } else if (op < 90) {                                 // finish a request
      const size_t k = rng() % live.size();
      if (pa_bm_free_request(bm, live[k].id) != PA_OK) ++errors;
      live[k] = live.back();
      live.pop_back();
    } else if (op < 95) {                                 // read its table back
      const Req &r = live[rng() % live.size()];
      if (pa_bm_table(bm, r.id, table, 512, &len) != PA_OK ||
          len != (r.len + kBlockSize - 1) / kBlockSize)
        ++errors;
      std::vector<uint64_t> ids;
      for (const Req &q : live) ids.push_back(q.id);
      std::vector<int32_t> tables(ids.size() * 512);
      if (pa_bm_fill_tables(bm, ids.data(), (int32_t)ids.size(), 512, tables.data()) != PA_OK)
        ++errors;
    } else {                                              // pool-wide reads
      int32_t nf, na, nr;
      if (pa_bm_stats(bm, &nf, &na, &nr) != PA_OK || nf + na != kBlocks) ++errors;
      if (pa_bm_free_ids(bm, free_ids, kBlocks, &len) != PA_OK) ++errors;
      (void)pa_bm_ref_count(bm, (int32_t)(rng() % kBlocks));
    }
  }
  for (const Req &r : live)
    if (pa_bm_free_request(bm, r.id) != PA_OK) ++errors;
  return errors;
}

}  // namespace

int main(int argc, char **argv) {
  const int threads = argc > 1 ? atoi(argv[1]) : 8;
  const int iters = argc > 2 ? atoi(argv[2]) : 20000;
  pa_block_manager *bm = nullptr;
  if (pa_bm_create(kBlocks, kBlockSize, &bm) != PA_OK) return 2;
  if (pa_bm_allocate(bm, kSystem, kSystemTokens, nullptr) != PA_OK) return 2;
  std::vector<int> errors(threads, 0);
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([&, t] { errors[t] = worker(bm, t, iters); });
  for (auto &th : pool) th.join();
  int bad = 0;
  for (int e : errors) bad += e;
  if (pa_bm_free_request(bm, kSystem) != PA_OK) ++bad;
  int32_t nf = -1, na = -1, nr = -1, len = -1;
  pa_bm_stats(bm, &nf, &na, &nr);
  if (nf != kBlocks || na != 0 || nr != 0) ++bad;
  std::vector<int32_t> ids(kBlocks);
  pa_bm_free_ids(bm, ids.data(), kBlocks, &len);
  std::vector<char> seen(kBlocks, 0);
  for (int32_t i = 0; i < len; ++i) {
    if (ids[i] < 0 || ids[i] >= kBlocks || seen[ids[i]]) ++bad;
    else seen[ids[i]] = 1;
  }
  for (int32_t b = 0; b < kBlocks; ++b)
    if (pa_bm_ref_count(bm, b) != 0) ++bad;
  pa_bm_destroy(bm);
  printf("bm_threads: %d threads x %d operations, free %d, allocated %d, requests %d, "
         "violations %d\n", threads, iters, nf, na, nr, bad);
  return bad == 0 ? 0 : 1;
}
