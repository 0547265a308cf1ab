// Host-pool driver for the sanitizer pass of the CPU tests: built with
// AddressSanitizer + UndefinedBehaviorSanitizer (leak detection on) together
// with csrc/pkv_host.cpp, it drives the block pool through its C ABI with
// seeded random operations -- create, fork, append (one or many tokens, and
// one token for a whole batch), free, prefix-cache hits and registrations,
// swap out and in, prefix groups, table checks, exhaustion and bad handles --
// and checks after every operation that
//   * each block's reference count equals the number of live sequences whose
//     table holds it,
//   * free + in use + cache-only (evictable) blocks = all blocks,
//   * a failed append leaves every table unchanged (all or nothing),
// then frees everything (every block back on the free list once the cache is
// cleared: the pages of cancelled requests return) and destroys the pool, so
// a leaked allocation fails the leak check at exit.
// Exit status 0 = all checks passed.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "pkv.h"

namespace {

int g_fail = 0;
// operations that took each path, over all seeds
int64_t g_swapped_out = 0, g_swapped_in = 0, g_cache_hits = 0, g_exhausted = 0, g_cow = 0,
        g_groups = 0;

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                            \
      return;                                                              \
    }                                                                      \
  } while (0)

std::vector<int32_t> table_of(const pkv_pool* p, int32_t seq) {
  int32_t n = 0;
  pkv_seq_block_table(p, seq, nullptr, 0, &n);
  std::vector<int32_t> t((size_t)n);
  if (n > 0) pkv_seq_block_table(p, seq, t.data(), n, &n);
  return t;
}

void check_invariants(const pkv_pool* p, int32_t nb, const std::vector<int32_t>& live) {
  std::vector<int32_t> holders((size_t)nb, 0);
  for (int32_t s : live)
    for (int32_t b : table_of(p, s))
      if (b >= 0) holders[(size_t)b] += 1;  // -1: swapped out
  int32_t in_use = 0;
  for (int32_t b = 0; b < nb; ++b) {
    CHECK(pkv_pool_refcount(p, b) == holders[(size_t)b]);
    in_use += holders[(size_t)b] > 0;
  }
  int32_t evictable = 0;
  CHECK(pkv_prefix_cache_stats(p, nullptr, nullptr, nullptr, &evictable) == PKV_OK);
  CHECK(pkv_pool_num_free(p) + in_use + evictable == nb);
}

std::vector<int32_t> prompt(std::mt19937& rng, int32_t family, int32_t n) {
  // prompts of one family share their first tokens, so the cache hits
  std::vector<int32_t> t((size_t)n);
  for (int32_t i = 0; i < n; ++i)
    t[(size_t)i] = i < 40 ? family * 1000 + i : (int32_t)(rng() % 50000);
  return t;
}

void run(uint32_t seed, int32_t nb, int n_ops) {
  std::mt19937 rng(seed);
  pkv_pool* p = nullptr;
  CHECK(pkv_pool_create(nb, 16, seed, &p) == PKV_OK && p != nullptr);
  CHECK(pkv_pool_set_swap_space(p, nb / 2) == PKV_OK);
  std::vector<int32_t> live;
  std::map<int32_t, std::vector<int32_t>> tokens;  // prompt of cache-created sequences
  for (int op = 0; op < n_ops; ++op) {
    const int kind = (int)(rng() % 10);
    const int32_t pick = live.empty() ? -1 : live[rng() % live.size()];
    if (kind == 0 || live.empty()) {
      int32_t s = -1;
      CHECK(pkv_seq_create(p, &s) == PKV_OK);
      live.push_back(s);
    } else if (kind == 1) {
      int32_t c = -1;
      const pkv_status st = pkv_seq_fork(p, pick, &c);
      if (st == PKV_OK) live.push_back(c);
      else CHECK(pkv_seq_num_swapped(p, pick) > 0);   // only a swapped parent refuses
    } else if (kind == 2 || kind == 3) {
      const int32_t n = (int32_t)(rng() % 70);
      std::vector<int64_t> slots((size_t)n + 1);
      int32_t cow[2], n_cow = 0;
      std::vector<std::vector<int32_t>> before;
      for (int32_t s : live) before.push_back(table_of(p, s));
      const pkv_status st = pkv_seq_append(p, pick, n, slots.data(), cow, &n_cow);
      g_exhausted += st == PKV_ERR_NO_FREE_BLOCKS;
      g_cow += st == PKV_OK && n_cow > 0;
      if (st != PKV_OK) {
        CHECK(st == PKV_ERR_NO_FREE_BLOCKS || pkv_seq_num_swapped(p, pick) > 0);
        for (size_t i = 0; i < live.size(); ++i) CHECK(table_of(p, live[i]) == before[i]);
      }
    } else if (kind == 4) {
      std::vector<int32_t> batch;
      for (int32_t s : live)
        if (pkv_seq_num_swapped(p, s) == 0 && rng() % 2) batch.push_back(s);
      std::vector<int64_t> slots(batch.size() + 1);
      std::vector<int32_t> cows(2 * batch.size() + 2);
      int32_t n_cow = 0, n_done = 0;
      const pkv_status st = pkv_seq_append_each(p, batch.data(), (int32_t)batch.size(),
                                                slots.data(), cows.data(), &n_cow, &n_done);
      CHECK(st == PKV_OK || st == PKV_ERR_NO_FREE_BLOCKS);
      CHECK(n_done <= (int32_t)batch.size() && n_cow <= n_done);
    } else if (kind == 5) {
      CHECK(pkv_seq_free(p, pick) == PKV_OK);
      for (size_t i = 0; i < live.size(); ++i)
        if (live[i] == pick) {
          live.erase(live.begin() + (long)i);
          break;
        }
      tokens.erase(pick);
      CHECK(pkv_seq_free(p, pick) == PKV_ERR_BAD_HANDLE);   // a second free is refused
    } else if (kind == 6) {
      const int32_t fam = (int32_t)(rng() % 3);
      std::vector<int32_t> t = prompt(rng, fam, 16 + (int32_t)(rng() % 80));
      int32_t s = -1, hit = 0;
      const pkv_status st = pkv_seq_create_cached(p, t.data(), (int32_t)t.size(), &s, &hit);
      if (st == PKV_OK) {
        live.push_back(s);
        CHECK(hit % 16 == 0 && hit <= (int32_t)t.size());
        g_cache_hits += hit > 0;
        std::vector<int64_t> slots(t.size() + 1);
        int32_t cow[2], n_cow = 0;
        if (pkv_seq_append(p, s, (int32_t)t.size() - hit, slots.data(), cow, &n_cow) ==
            PKV_OK) {
          CHECK(pkv_seq_cache_prefix(p, s, t.data(), (int32_t)t.size()) == PKV_OK);
          tokens[s] = t;
        }
      } else {
        CHECK(st == PKV_ERR_NO_FREE_BLOCKS);
      }
    } else if (kind == 7) {
      const int32_t n = (int32_t)table_of(p, pick).size();
      if (n > 0 && pkv_seq_num_swapped(p, pick) == 0) {
        const int32_t first = (int32_t)(rng() % n), cnt = 1 + (int32_t)(rng() % (n - first));
        std::vector<int32_t> pairs(2 * (size_t)cnt);
        const pkv_status st = pkv_seq_swap_out(p, pick, first, cnt, pairs.data());
        CHECK(st == PKV_OK || st == PKV_ERR_REFCOUNT || st == PKV_ERR_NO_FREE_BLOCKS);
        g_swapped_out += st == PKV_OK;
      }
    } else if (kind == 8) {
      for (int32_t s : live)
        if (pkv_seq_num_swapped(p, s) > 0) {
          int32_t n = 0;
          pkv_seq_swap_in(p, s, nullptr, 0, &n);
          std::vector<int32_t> pairs(2 * (size_t)n + 2);
          const pkv_status st = pkv_seq_swap_in(p, s, pairs.data(), n, &n);
          CHECK(st == PKV_OK || st == PKV_ERR_NO_FREE_BLOCKS);
          g_swapped_in += st == PKV_OK;
          break;
        }
    } else {
      // prefix groups of the live, resident sequences and the host table check
      std::vector<int32_t> batch;
      for (int32_t s : live)
        if (pkv_seq_num_swapped(p, s) == 0) batch.push_back(s);
      const int32_t n = (int32_t)batch.size();
      std::vector<int32_t> pre((size_t)n + 1), groups(((size_t)n + 1) * 4), order((size_t)n + 1);
      int32_t ng = 0, mp = 0;
      const pkv_status st = pkv_pool_prefix_groups(p, batch.data(), n, 4, n + 1, pre.data(),
                                                   groups.data(), &ng, &mp, order.data());
      CHECK(st == PKV_OK);
      g_groups += ng;
      // the cascade's tail count and its listed units agree, in pool order
      int64_t units = 0, listed = -1;
      CHECK(pkv_pool_cascade_tail_units(p, batch.data(), n, pre.data(), mp, 32, &units) ==
            PKV_OK);
      std::vector<int32_t> tmap((size_t)units * 2 + 2);
      CHECK(pkv_pool_cascade_tail_map(p, batch.data(), n, pre.data(), mp, 32, order.data(),
                                      tmap.data(), units, &listed) == PKV_OK);
      CHECK(listed == units);
      if (units > 0)   // one unit short: refused
        CHECK(pkv_pool_cascade_tail_map(p, batch.data(), n, pre.data(), mp, 32, order.data(),
                                        tmap.data(), units - 1, &listed) ==
              PKV_ERR_INVALID_ARG);
      int32_t width = 1;
      for (int32_t s : batch) width = std::max<int32_t>(width, (int32_t)table_of(p, s).size());
      std::vector<int32_t> tables((size_t)n * (size_t)width + 1, 0), lens((size_t)n + 1, 0);
      for (int32_t i = 0; i < n; ++i) {
        const std::vector<int32_t> t = table_of(p, batch[(size_t)i]);
        for (size_t j = 0; j < t.size(); ++j) tables[(size_t)i * width + j] = t[j];
        lens[(size_t)i] = (int32_t)pkv_seq_len(p, batch[(size_t)i]);
      }
      int32_t bad = 0;
      CHECK(pkv_validate_tables(tables.data(), width, lens.data(), n, width * 16, nb, &bad) ==
            PKV_OK);
      CHECK(bad == -1);
    }
    check_invariants(p, nb, live);
    if (g_fail) break;
  }
  // cancel everything: every page returns ([GLOSSARY] §4.02)
  for (int32_t s : live) CHECK(pkv_seq_free(p, s) == PKV_OK);
  pkv_prefix_cache_clear(p);
  CHECK(pkv_pool_num_free(p) == nb);
  CHECK(pkv_pool_num_free_host(p) == nb / 2);
  std::vector<int32_t> none;
  check_invariants(p, nb, none);
  pkv_pool_destroy(p);
  CHECK(pkv_seq_create(nullptr, nullptr) == PKV_ERR_BAD_HANDLE);
}

}  // namespace

int main() {
  for (uint32_t seed = 1; seed <= 6; ++seed) run(seed, 24 + 16 * (int32_t)seed, 1500);
  std::printf("paths taken: swap out %lld, swap in %lld, cache hits %lld, exhausted %lld, "
              "copy-on-write %lld, prefix groups %lld\n",
              (long long)g_swapped_out, (long long)g_swapped_in, (long long)g_cache_hits,
              (long long)g_exhausted, (long long)g_cow, (long long)g_groups);
  if (!g_swapped_out || !g_swapped_in || !g_cache_hits || !g_exhausted || !g_cow || !g_groups) {
    std::fprintf(stderr, "a path was never taken\n");
    ++g_fail;
  }
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("pool driver: all checks passed\n");
  return 0;
}
