// Stress of the host page allocator (pkv_pages.cpp) built alone with g++ and sanitizers: random
// forks, growth, releases, prefix inserts / lookups and evictions, with the reference counts
// recounted from the sequences' tables after every step.
#include <cstdio>
#include <random>
#include <vector>

#include "../../include/pkv.h"

int main() {
  const int NP = 48, PS = 4;
  pkv_page_allocator* a = pkv_pages_create(NP, PS);
  if (!a) return 1;
  std::mt19937 rng(7);
  std::vector<int32_t> live;
  std::vector<std::vector<int32_t>> toks(4096);
  int failures = 0;
  for (int step = 0; step < 3000; ++step) {
    const int op = int(rng() % 7);
    int32_t sid = -1, n = 0, copies[2], nc = 0, matched = 0, ev = 0;
    if (op == 0 || live.empty()) {
      pkv_pages_seq_create(a, &sid);
      live.push_back(sid);
      toks[sid].clear();
    } else if (op == 1) {
      const int32_t src = live[rng() % live.size()];
      pkv_pages_seq_fork(a, src, &sid);
      live.push_back(sid);
      toks[sid] = toks[src];
    } else if (op == 2) {
      const size_t i = rng() % live.size();
      pkv_pages_seq_release(a, live[i]);
      live.erase(live.begin() + long(i));
    } else if (op == 3) {
      sid = live[rng() % live.size()];
      n = int32_t(rng() % 9);
      if (pkv_pages_seq_reserve(a, sid, n, copies, 1, &nc) == PKV_OK)
        for (int i = 0; i < n; ++i) toks[sid].push_back(int32_t(rng() % 3));
    } else if (op == 4) {
      sid = live[rng() % live.size()];
      pkv_pages_prefix_insert(a, sid, toks[sid].data(), int32_t(toks[sid].size()));
    } else if (op == 5) {
      const std::vector<int32_t>& src = toks[live[rng() % live.size()]];
      if (pkv_pages_seq_create_with_prefix(a, src.data(), int32_t(src.size()), &sid, &matched) == PKV_OK) {
        live.push_back(sid);
        toks[sid].assign(src.begin(), src.begin() + matched);
      }
    } else {
      pkv_pages_prefix_evict(a, int32_t(rng() % 3), &ev);
    }
    // every live sequence's pages are referenced, and the free count is consistent
    std::vector<int> seen(NP, 0);
    for (int32_t s : live) {
      int32_t row[64], np = 0;
      if (pkv_pages_seq_table(a, s, row, 64, &np) != PKV_OK) { ++failures; continue; }
      for (int i = 0; i < np; ++i) ++seen[row[i]];
    }
    int free_pages = 0;
    for (int p = 0; p < NP; ++p) {
      if (pkv_pages_refcount(a, p) < seen[p]) ++failures;
      if (pkv_pages_refcount(a, p) == 0) ++free_pages;
    }
    if (free_pages != pkv_pages_free_count(a)) ++failures;
  }
  pkv_pages_destroy(a);
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("all checks passed\n");
  return 0;
}
