// Random operation streams through the block manager's C API, for a host
// build with AddressSanitizer and UndefinedBehaviorSanitizer: every status
// path runs, and after each operation the reference counts must be valid,
// referenced plus free blocks must equal each pool, and every live
// sequence's table must read back.
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <vector>
#include <random>
#include <set>
#include "pkv_blocks.h"

int main(int argc, char **argv) {
  const int trials = argc > 1 ? atoi(argv[1]) : 200;
  std::mt19937_64 rng(12345);
  long ops = 0, errs = 0;
  for (int trial = 0; trial < trials; ++trial) {
    const int NB = 1 + rng() % 64, NH = rng() % 48, BS = 1 + rng() % 17;
    pkv_block_manager *bm = nullptr;
    if (pkv_bm_create_with_host(NB, NH, BS, &bm) != 0) { printf("create failed\n"); return 1; }
    std::set<int64_t> live;
    int64_t next_id = 0;
    for (int step = 0; step < 400; ++step, ++ops) {
      const int op = rng() % 7;
      std::vector<int64_t> ids;
      for (auto x : live) if (rng() % 3 == 0) ids.push_back(x);
      if (ids.empty() && !live.empty()) ids.push_back(*live.begin());
      int rc = 0;
      if (op == 0) {
        std::vector<int64_t> slots(200);
        const int nt = rng() % 40;
        rc = pkv_bm_add_sequence(bm, next_id, nt, slots.data());
        if (rc == 0) live.insert(next_id);
        ++next_id;
      } else if (op == 1 && !live.empty()) {
        rc = pkv_bm_fork(bm, *live.rbegin(), next_id);
        if (rc == 0) live.insert(next_id);
        ++next_id;
      } else if (op == 2 && !ids.empty()) {
        const int n = (int)ids.size();
        std::vector<int64_t> slots(n), pairs(2 * n);
        int32_t nc = -1;
        rc = pkv_bm_append_tokens(bm, ids.data(), n, slots.data(), pairs.data(), &nc);
      } else if (op == 3 && !ids.empty()) {
        rc = pkv_bm_free_sequence(bm, ids[0]);
        if (rc == 0) live.erase(ids[0]);
      } else if (op == 4 && !ids.empty()) {
        std::vector<int64_t> pairs(2 * 512);
        int32_t np = -1;
        rc = pkv_bm_swap_out(bm, ids.data(), (int)ids.size(), pairs.data(), 512, &np);
      } else if (op == 5 && !ids.empty()) {
        std::vector<int64_t> pairs(2 * 512);
        int32_t np = -1;
        rc = pkv_bm_swap_in(bm, ids.data(), (int)ids.size(), pairs.data(), 512, &np);
      } else if (op == 6 && !ids.empty()) {
        const int n = (int)ids.size(), mb = 1 + rng() % 16;
        std::vector<int32_t> tables(n * mb), lens(n);
        rc = pkv_bm_batch_tables(bm, ids.data(), n, mb, tables.data(), lens.data());
      }
      if (rc != 0) ++errs;
      // invariants: refcounts non-negative and free + referenced = pool size
      int used = 0, hused = 0;
      for (int b = 0; b < NB; ++b) { const int r = pkv_bm_refcount(bm, b); if (r < 0) { printf("bad ref\n"); return 1; } used += r > 0; }
      for (int b = 0; b < NH; ++b) { const int r = pkv_bm_host_refcount(bm, b); if (r < 0) { printf("bad href\n"); return 1; } hused += r > 0; }
      if (used + pkv_bm_num_free_blocks(bm) != NB || hused + pkv_bm_num_free_host_blocks(bm) != NH) {
        printf("pool accounting broken: trial %d step %d\n", trial, step); return 1;
      }
      for (auto x : live) {
        std::vector<int32_t> t(4096); int32_t nb = -1;
        if (pkv_bm_block_table(bm, x, t.data(), 4096, &nb) != 0) { printf("table failed\n"); return 1; }
        if (pkv_bm_num_tokens(bm, x) < 0) { printf("tokens\n"); return 1; }
      }
    }
    pkv_bm_destroy(bm);
  }
  printf("ok: %ld operations, %ld refused with a status\n", ops, errs);
  return 0;
}
