// Host allocator driver for the sanitizer tests (test infrastructure; built
// with g++ for the host only).
//
//   alloc_fuzz            random operation sequences on one thread; after
//                         every operation each page's reference count must
//                         equal the number of tables and cache entries that
//                         hold it, and the free pages must be exactly those
//                         with count 0; then block-table validation on
//                         random tables.
//   alloc_fuzz threads    eight threads issuing random operations on one
//                         shared allocator (the calls serialise on its
//                         lock), then the same invariant once they are done.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <thread>
#include <vector>
#include "pkv.h"

static int check_invariant(pkv_allocator* a, int N, int S, std::vector<int32_t>& pages) {
  std::vector<int> held(N, 0);
  for (int s = 0; s < S; ++s) {
    int32_t tab[64];
    int32_t np = 0;
    if (pkv_alloc_table(a, s, tab, 64, &np) != PKV_OK) return 1;
    for (int j = 0; j < np; ++j) held[tab[j]] += 1;
  }
  for (int k = 0; k < 4; ++k) {
    int32_t np = 0, nt = 0;
    if (pkv_alloc_cache_lookup(a, k, pages.data(), N, &np, &nt) == PKV_OK)
      for (int j = 0; j < np; ++j) held[pages[j]] += 1;
  }
  int free_pages = 0;
  for (int p = 0; p < N; ++p) {
    int32_t c = -1;
    pkv_alloc_refcount(a, p, &c);
    if (c != held[p]) {
      printf("page %d refcount %d held %d\n", p, c, held[p]);
      return 1;
    }
    if (c == 0) ++free_pages;
  }
  if (free_pages != pkv_alloc_free_count(a)) {
    printf("free count mismatch\n");
    return 1;
  }
  return 0;
}

static void random_op(pkv_allocator* a, std::mt19937& rng, int N, int P, int S, int W) {
  std::vector<int32_t> bt(S * W), src(S * W + 8), dst(S * W + 8), pages(N);
  const int kind = rng() % 8;
  const int32_t seq = rng() % S;
  if (kind == 0) {
    int32_t np;
    pkv_alloc_reserve(a, seq, rng() % (W * P + 5), bt.data(), W, &np);
  } else if (kind == 1) {
    const int32_t B = 1 + rng() % S;
    std::vector<int32_t> seqs, nt;
    for (int i = 0; i < B; ++i) {
      seqs.push_back(rng() % S);
      nt.push_back(rng() % (W * P));
    }
    pkv_alloc_reserve_batch(a, B, seqs.data(), nt.data(), bt.data(), W);
  } else if (kind == 2) {
    pkv_alloc_free(a, seq);
  } else if (kind == 3) {
    int32_t np = 0, tab[64];
    if (pkv_alloc_table(a, (seq + 1) % S, tab, 64, &np) == PKV_OK && np > 0) pkv_alloc_share_prefix(a, seq, tab, np);
  } else if (kind == 4) {
    pkv_alloc_cache_insert(a, rng() % 4, seq, 1 + rng() % (W * P));
  } else if (kind == 5) {
    int32_t np, nt;
    pkv_alloc_cache_lookup(a, rng() % 4, pages.data(), N, &np, &nt);
  } else if (kind == 6) {
    pkv_alloc_cache_evict(a, rng() % 4);
  } else {
    const int32_t B = 1 + rng() % S;
    std::vector<int32_t> seqs, pos;
    int32_t nc = 0;
    for (int i = 0; i < B; ++i) {
      seqs.push_back(rng() % S);
      pos.push_back(rng() % (W * P));
    }
    pkv_alloc_prepare_append(a, B, seqs.data(), pos.data(), src.data(), dst.data(), &nc, bt.data(), W);
  }
}

static int threaded() {
  const int N = 48, P = 16, S = 8, W = 12;
  pkv_allocator* a = nullptr;
  if (pkv_alloc_create(N, P, nullptr, &a) != PKV_OK) return 1;
  std::vector<std::thread> pool;
  for (int t = 0; t < 8; ++t)
    pool.emplace_back([a, t] {
      std::mt19937 rng(100 + t);
      for (int op = 0; op < 2000; ++op) random_op(a, rng, N, P, S, W);
    });
  for (auto& th : pool) th.join();
  std::vector<int32_t> pages(N);
  const int rc = check_invariant(a, N, S, pages);
  pkv_alloc_destroy(a);
  return rc;
}

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "threads") == 0) {
    const int rc = threaded();
    printf(rc ? "FAILED\n" : "ok\n");
    return rc;
  }
  std::mt19937 rng(1234);
  for (int trial = 0; trial < 300; ++trial) {
    const int N = 1 + rng() % 64, P = 16 << (rng() % 3), S = 1 + rng() % 8, W = 1 + rng() % 16;
    pkv_allocator* a = nullptr;
    if (pkv_alloc_create(N, P, nullptr, &a) != PKV_OK) { printf("create failed\n"); return 1; }
    std::vector<int32_t> pages(N);
    for (int op = 0; op < 200; ++op) {
      random_op(a, rng, N, P, S, W);
      if (check_invariant(a, N, S, pages)) {
        printf("trial %d op %d\n", trial, op);
        return 1;
      }
    }
    pkv_alloc_destroy(a);
  }
  // validate_tables on random garbage
  for (int t = 0; t < 2000; ++t) {
    int B = rng() % 6, W = rng() % 5, P = 16, N = rng() % 10;
    std::vector<int32_t> bt(B * W + 1), lens(B + 1);
    for (auto& x : bt) x = (int32_t)(rng() % 14) - 2;
    for (auto& x : lens) x = (int32_t)(rng() % 100) - 5;
    int32_t r, e, rule;
    // plain tables, shared prefixes (up to 2 pages) and rings (windows up to 70 tokens; lengths far past the ring)
    const int mode = rng() % 3;
    const int32_t prefix = mode == 1 ? (int32_t)(rng() % 3) * P : 0;
    const int32_t window = mode == 2 ? (int32_t)(rng() % 70) : 0;
    if (mode == 2)
      for (auto& x : lens) x = (int32_t)(rng() % 400) - 5;
    pkv_validate_tables(bt.data(), lens.data(), B, W, P, N, rng() % 2, prefix, window, &r, &e, &rule);
  }
  printf("ok\n");
  return 0;
}
