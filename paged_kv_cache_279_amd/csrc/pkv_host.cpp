// Host side of libpkv: status strings, the page allocator and block-table
// validation. Plain C++17, no device calls.
//
// The allocator keeps the page table in native code with the scheduling
// policy above it (pgsm §4.3 notes that serving stacks keep the page table in
// C/C++ and only schedule from Python). Pages are handed out on demand and
// returned when a request ends or fails (dpshk §4.2); a shared system-prompt
// prefix is stored once and referenced by every sequence that uses it
// (dpshk §4.2, pgsm §3.2).

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <memory>
#include <mutex>
#include <new>
#include <stdexcept>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv.h"

struct pkv_cache_entry {
  std::vector<int32_t> pages;
  int32_t n_tokens = 0;
  uint64_t last_use = 0;                         // allocator clock at the last insert / lookup
};

struct pkv_allocator {
  int32_t num_pages = 0;
  int32_t page_size = 0;
  std::deque<int32_t> free_list;                 // FIFO: pop front, push back
  std::vector<int32_t> refcount;                 // per page: tables + cache entries holding it
  std::unordered_map<int32_t, std::vector<int32_t>> tables;
  std::unordered_map<uint64_t, pkv_cache_entry> cache;   // prefix cache
  uint64_t clock = 0;
  mutable std::mutex mu;
};

namespace {

int64_t pages_for(int64_t tokens, int32_t page_size) { return (tokens + page_size - 1) / page_size; }

// Run an entry point's body; a failed host allocation inside it becomes a
// status code instead of an exception crossing the C interface.
template <class F>
int guarded(F&& body) noexcept {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return PKV_ERR_HOST_MEMORY;
  } catch (const std::length_error&) {
    return PKV_ERR_HOST_MEMORY;
  }
}

void write_row(const std::vector<int32_t>& pages, int32_t* row, int32_t max_pages) {
  if (!row) return;
  const int32_t n = static_cast<int32_t>(pages.size());
  for (int32_t j = 0; j < max_pages; ++j) row[j] = j < n ? pages[j] : -1;
}

void release(pkv_allocator* a, const std::vector<int32_t>& pages) {
  for (int32_t p : pages) {
    if (--a->refcount[p] == 0) a->free_list.push_back(p);
  }
}

// Prefix-cache eviction: drop least recently used entries until `need` pages
// are free, if dropping every entry would free enough (pages held only by the
// cache); otherwise change nothing. Callers hold the lock.
bool make_room(pkv_allocator* a, int64_t need) {
  if (need <= static_cast<int64_t>(a->free_list.size())) return true;
  std::unordered_map<int32_t, int32_t> held;
  for (const auto& kv : a->cache)
    for (int32_t p : kv.second.pages) held[p] += 1;
  int64_t freeable = 0;
  for (const auto& kv : held)
    if (a->refcount[kv.first] == kv.second) freeable += 1;
  if (need > static_cast<int64_t>(a->free_list.size()) + freeable) return false;
  std::vector<std::pair<uint64_t, uint64_t>> order;   // (last use, key)
  order.reserve(a->cache.size());
  for (const auto& kv : a->cache) order.emplace_back(kv.second.last_use, kv.first);
  std::sort(order.begin(), order.end());
  for (const auto& o : order) {
    if (need <= static_cast<int64_t>(a->free_list.size())) break;
    auto it = a->cache.find(o.second);
    release(a, it->second.pages);
    a->cache.erase(it);
  }
  return true;
}

// Grow `seq`'s table to `want` pages from the front of the free list (room
// already made). Callers hold the lock.
void grow(pkv_allocator* a, int32_t seq, int64_t want) {
  std::vector<int32_t>& tab = a->tables[seq];
  while (static_cast<int64_t>(tab.size()) < want) {
    const int32_t p = a->free_list.front();
    a->free_list.pop_front();
    a->refcount[p] = 1;
    tab.push_back(p);
  }
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_OUT_OF_PAGES: return "PKV_ERR_OUT_OF_PAGES";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "PKV_ERR_WORKSPACE_TOO_SMALL";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_INVALID_TABLE: return "PKV_ERR_INVALID_TABLE";
    case PKV_ERR_NOT_FOUND: return "PKV_ERR_NOT_FOUND";
    case PKV_ERR_HOST_MEMORY: return "PKV_ERR_HOST_MEMORY";
    case PKV_ERR_SCRATCH_LIMIT: return "PKV_ERR_SCRATCH_LIMIT";
    default: return "PKV_ERR_UNKNOWN";
  }
}

int pkv_abi_version(void) { return 2; }

int pkv_alloc_create(int32_t num_pages, int32_t page_size, const int32_t* free_order,
                     pkv_allocator** out) {
  return guarded([&]() -> int {
    if (!out || num_pages < 0 || page_size <= 0) return PKV_ERR_INVALID_ARG;
    *out = nullptr;
    std::vector<int32_t> order(static_cast<size_t>(num_pages));
    if (free_order) {
      std::vector<char> seen(static_cast<size_t>(num_pages), 0);
      for (int32_t i = 0; i < num_pages; ++i) {
        const int32_t p = free_order[i];
        if (p < 0 || p >= num_pages || seen[p]) return PKV_ERR_INVALID_ARG;
        seen[p] = 1;
        order[i] = p;
      }
    } else {
      for (int32_t i = 0; i < num_pages; ++i) order[i] = i;
    }
    std::unique_ptr<pkv_allocator> a(new pkv_allocator());
    a->num_pages = num_pages;
    a->page_size = page_size;
    a->free_list.assign(order.begin(), order.end());
    a->refcount.assign(static_cast<size_t>(num_pages), 0);
    *out = a.release();
    return PKV_OK;
  });
}

void pkv_alloc_destroy(pkv_allocator* alloc) { delete alloc; }

int pkv_alloc_reserve_batch(pkv_allocator* a, int32_t B, const int32_t* seqs, const int32_t* n_tokens,
                            int32_t* block_table, int32_t max_pages) {
  return guarded([&]() -> int {
    if (!a || B < 0 || (B > 0 && (!seqs || !n_tokens))) return PKV_ERR_INVALID_ARG;
    if (block_table && max_pages < 0) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(a->mu);
    // plan first, touch nothing until the whole batch fits
    int64_t need_total = 0;
    std::unordered_set<int32_t> in_batch;
    for (int32_t i = 0; i < B; ++i) {
      if (seqs[i] < 0 || n_tokens[i] < 0 || !in_batch.insert(seqs[i]).second) return PKV_ERR_INVALID_ARG;
      const int64_t want = pages_for(n_tokens[i], a->page_size);
      auto tab = a->tables.find(seqs[i]);
      const int64_t have = tab == a->tables.end() ? 0 : static_cast<int64_t>(tab->second.size());
      if (block_table && std::max(want, have) > max_pages) return PKV_ERR_INVALID_ARG;
      need_total += std::max<int64_t>(0, want - have);
    }
    if (!make_room(a, need_total)) return PKV_ERR_OUT_OF_PAGES;
    // commit: pages leave the free list in batch order
    for (int32_t i = 0; i < B; ++i) grow(a, seqs[i], pages_for(n_tokens[i], a->page_size));
    if (block_table) {
      for (int32_t i = 0; i < B; ++i)
        write_row(a->tables[seqs[i]], block_table + static_cast<int64_t>(i) * max_pages, max_pages);
    }
    return PKV_OK;
  });
}

int pkv_alloc_reserve(pkv_allocator* a, int32_t seq, int32_t n_tokens, int32_t* bt_row,
                      int32_t max_pages, int32_t* n_pages) {
  return guarded([&]() -> int {
    if (!a) return PKV_ERR_INVALID_ARG;
    const int rc = pkv_alloc_reserve_batch(a, 1, &seq, &n_tokens, bt_row, max_pages);
    if (rc == PKV_OK && n_pages) {
      std::lock_guard<std::mutex> lock(a->mu);
      *n_pages = static_cast<int32_t>(a->tables[seq].size());
    }
    return rc;
  });
}

int pkv_alloc_share_prefix(pkv_allocator* a, int32_t seq, const int32_t* pages, int32_t n) {
  return guarded([&]() -> int {
    if (!a || seq < 0 || n < 0 || (n > 0 && !pages)) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(a->mu);
    auto tab = a->tables.find(seq);
    if (tab != a->tables.end() && !tab->second.empty()) return PKV_ERR_INVALID_ARG;
    std::unordered_set<int32_t> seen;
    for (int32_t i = 0; i < n; ++i) {
      const int32_t p = pages[i];
      if (p < 0 || p >= a->num_pages || a->refcount[p] <= 0 || !seen.insert(p).second)
        return PKV_ERR_INVALID_ARG;
    }
    std::vector<int32_t>& t = a->tables[seq];
    t.assign(pages, pages + n);
    for (int32_t i = 0; i < n; ++i) a->refcount[pages[i]] += 1;
    return PKV_OK;
  });
}

int pkv_alloc_free(pkv_allocator* a, int32_t seq) {
  return guarded([&]() -> int {
    if (!a) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(a->mu);
    auto tab = a->tables.find(seq);
    if (tab == a->tables.end()) return PKV_OK;
    release(a, tab->second);
    a->tables.erase(tab);
    return PKV_OK;
  });
}

int pkv_alloc_cache_insert(pkv_allocator* a, uint64_t key, int32_t seq, int32_t n_tokens) {
  return guarded([&]() -> int {
    if (!a || n_tokens <= 0) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(a->mu);
    auto tab = a->tables.find(seq);
    const int64_t n_pages = pages_for(n_tokens, a->page_size);
    if (tab == a->tables.end() || n_pages > static_cast<int64_t>(tab->second.size())) return PKV_ERR_INVALID_ARG;
    auto it = a->cache.find(key);
    if (it != a->cache.end()) {
      it->second.last_use = ++a->clock;
      return PKV_OK;
    }
    pkv_cache_entry e;
    e.pages.assign(tab->second.begin(), tab->second.begin() + n_pages);
    for (int32_t p : e.pages) a->refcount[p] += 1;
    e.n_tokens = n_tokens;
    e.last_use = ++a->clock;
    a->cache.emplace(key, std::move(e));
    return PKV_OK;
  });
}

int pkv_alloc_cache_lookup(pkv_allocator* a, uint64_t key, int32_t* pages, int32_t max_pages, int32_t* n_pages,
                           int32_t* n_tokens) {
  return guarded([&]() -> int {
    if (!a || max_pages < 0 || (max_pages > 0 && !pages)) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(a->mu);
    auto it = a->cache.find(key);
    if (it == a->cache.end()) return PKV_ERR_NOT_FOUND;
    const pkv_cache_entry& e = it->second;
    if (pages && static_cast<int64_t>(e.pages.size()) > max_pages) return PKV_ERR_INVALID_ARG;
    it->second.last_use = ++a->clock;
    if (pages) std::copy(e.pages.begin(), e.pages.end(), pages);
    if (n_pages) *n_pages = static_cast<int32_t>(e.pages.size());
    if (n_tokens) *n_tokens = e.n_tokens;
    return PKV_OK;
  });
}

int pkv_alloc_cache_evict(pkv_allocator* a, uint64_t key) {
  return guarded([&]() -> int {
    if (!a) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(a->mu);
    auto it = a->cache.find(key);
    if (it == a->cache.end()) return PKV_OK;
    release(a, it->second.pages);
    a->cache.erase(it);
    return PKV_OK;
  });
}

int32_t pkv_alloc_cache_entries(const pkv_allocator* a) {
  if (!a) return -1;
  std::lock_guard<std::mutex> lock(a->mu);
  return static_cast<int32_t>(a->cache.size());
}

int pkv_alloc_prepare_append(pkv_allocator* a, int32_t B, const int32_t* seqs, const int32_t* pos,
                             int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies, int32_t* block_table,
                             int32_t max_pages) {
  return guarded([&]() -> int {
    if (!a || B < 0 || (B > 0 && (!seqs || !pos || !copy_src || !copy_dst)) || !n_copies) return PKV_ERR_INVALID_ARG;
    if (block_table && max_pages < 0) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(a->mu);
    // plan with the counts as they stand: new pages to grow into, plus one per shared page written
    int64_t need = 0;
    std::unordered_set<int32_t> in_batch;
    for (int32_t i = 0; i < B; ++i) {
      if (seqs[i] < 0 || pos[i] < 0 || !in_batch.insert(seqs[i]).second) return PKV_ERR_INVALID_ARG;
      auto tab = a->tables.find(seqs[i]);
      const int64_t have = tab == a->tables.end() ? 0 : static_cast<int64_t>(tab->second.size());
      const int64_t j = pos[i] / a->page_size;
      if (block_table && std::max(j + 1, have) > max_pages) return PKV_ERR_INVALID_ARG;
      need += std::max<int64_t>(0, j + 1 - have);
      if (j < have && a->refcount[tab->second[j]] > 1) need += 1;
    }
    if (!make_room(a, need)) return PKV_ERR_OUT_OF_PAGES;
    int32_t n = 0;
    for (int32_t i = 0; i < B; ++i) {
      const int64_t j = pos[i] / a->page_size;
      grow(a, seqs[i], j + 1);
      std::vector<int32_t>& tab = a->tables[seqs[i]];
      const int32_t old = tab[j];
      if (a->refcount[old] > 1) {
        const int32_t fresh = a->free_list.front();
        a->free_list.pop_front();
        a->refcount[fresh] = 1;
        a->refcount[old] -= 1;
        tab[j] = fresh;
        copy_src[n] = old;
        copy_dst[n] = fresh;
        ++n;
      }
    }
    *n_copies = n;
    if (block_table) {
      for (int32_t i = 0; i < B; ++i)
        write_row(a->tables[seqs[i]], block_table + static_cast<int64_t>(i) * max_pages, max_pages);
    }
    return PKV_OK;
  });
}

int32_t pkv_alloc_free_count(const pkv_allocator* a) {
  if (!a) return -1;
  std::lock_guard<std::mutex> lock(a->mu);
  return static_cast<int32_t>(a->free_list.size());
}

int pkv_alloc_table(const pkv_allocator* a, int32_t seq, int32_t* bt_row, int32_t max_pages,
                    int32_t* n_pages) {
  if (!a || max_pages < 0 || (max_pages > 0 && !bt_row)) return PKV_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(a->mu);
  auto tab = a->tables.find(seq);
  static const std::vector<int32_t> kEmpty;
  const std::vector<int32_t>& pages = tab == a->tables.end() ? kEmpty : tab->second;
  if (static_cast<int64_t>(pages.size()) > max_pages && bt_row) return PKV_ERR_INVALID_ARG;
  write_row(pages, bt_row, max_pages);
  if (n_pages) *n_pages = static_cast<int32_t>(pages.size());
  return PKV_OK;
}

int pkv_alloc_refcount(const pkv_allocator* a, int32_t page, int32_t* count) {
  if (!a || !count) return PKV_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(a->mu);
  if (page < 0 || page >= a->num_pages) return PKV_ERR_INVALID_ARG;
  *count = a->refcount[page];
  return PKV_OK;
}

int pkv_validate_tables(const int32_t* bt, const int32_t* lens, int32_t B, int32_t max_pages, int32_t P,
                        int32_t N, int32_t exclusive_tail, int32_t prefix_tokens, int32_t window, int32_t* bad_row,
                        int32_t* bad_entry, int32_t* rule) {
  return guarded([&]() -> int {
    if (B < 0 || max_pages < 0 || P <= 0 || N < 0 || prefix_tokens < 0 || window < 0) return PKV_ERR_INVALID_ARG;
    if (prefix_tokens % P != 0 || (window > 0 && prefix_tokens > 0)) return PKV_ERR_INVALID_ARG;
    // a window must fit its ring: the pages it touches are distinct entries
    if (window > 0 && static_cast<int64_t>(window) > (static_cast<int64_t>(max_pages) - 1) * P + 1)
      return PKV_ERR_INVALID_ARG;
    if (B > 0 && (!bt || !lens)) return PKV_ERR_INVALID_ARG;
    auto fail = [&](int32_t r, int32_t row, int32_t entry) {
      if (bad_row) *bad_row = row;
      if (bad_entry) *bad_entry = entry;
      if (rule) *rule = r;
      return PKV_ERR_INVALID_TABLE;
    };
    if (bad_row) *bad_row = -1;
    if (bad_entry) *bad_entry = -1;
    if (rule) *rule = 0;
    // the entries a row's tokens reach, in token order: logical pages 0 ..
    // ceil(L / P) - 1, or under a window the ring entries (j % max_pages) of
    // the logical pages holding tokens max(0, L - window) .. L - 1
    auto reached = [&](int64_t L, std::vector<int32_t>& out) {
      out.clear();
      if (L <= 0) return;
      const int64_t lo = window > 0 ? std::max<int64_t>(0, L - window) : 0;
      for (int64_t j = lo / P; j <= (L - 1) / P; ++j)
        out.push_back(static_cast<int32_t>(window > 0 ? j % max_pages : j));
    };
    std::vector<int32_t> owners(static_cast<size_t>(N), 0);   // rows referencing each page
    std::vector<int32_t> last_owner(static_cast<size_t>(N), -1);
    std::vector<int32_t> mark(static_cast<size_t>(N), -1);     // row that last saw the page
    std::vector<int32_t> tail(static_cast<size_t>(B), -1);     // entry of each row's last token
    std::vector<int32_t> ent;
    for (int32_t b = 0; b < B; ++b) {
      const int64_t n = lens[b];
      if (n < 0) return fail(1, b, -1);
      if (window == 0 && pages_for(n, P) > max_pages) return fail(2, b, -1);
      reached(n, ent);
      const int32_t* row = bt + static_cast<int64_t>(b) * max_pages;
      for (const int32_t j : ent) {
        const int32_t p = row[j];
        if (p < 0 || p >= N) return fail(3, b, j);
        if (mark[p] == b) return fail(4, b, j);
        mark[p] = b;
        if (last_owner[p] != b) {
          owners[p] += 1;
          last_owner[p] = b;
        }
      }
      if (!ent.empty()) tail[b] = ent.back();
    }
    if (exclusive_tail) {
      for (int32_t b = 0; b < B; ++b) {
        if (tail[b] < 0) continue;
        const int32_t p = bt[static_cast<int64_t>(b) * max_pages + tail[b]];
        if (owners[p] > 1) return fail(5, b, tail[b]);
      }
    }
    if (prefix_tokens > 0) {
      // every attended row (lens > 0) holds the shared prefix in the same pages
      // as the first attended row; an idle row (lens == 0) may hold anything
      const int32_t np = prefix_tokens / P;
      int32_t first = -1;
      for (int32_t b = 0; b < B; ++b) {
        if (lens[b] == 0) continue;
        if (lens[b] < prefix_tokens) return fail(7, b, -1);
        if (first < 0) {
          first = b;
          continue;
        }
        const int32_t* row = bt + static_cast<int64_t>(b) * max_pages;
        const int32_t* ref = bt + static_cast<int64_t>(first) * max_pages;
        for (int32_t j = 0; j < np; ++j)
          if (row[j] != ref[j]) return fail(6, b, j);
      }
    }
    return PKV_OK;
  });
}

}  // extern "C"
