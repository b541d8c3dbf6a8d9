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
#include <mutex>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv.h"

struct pkv_allocator {
  int32_t num_pages = 0;
  int32_t page_size = 0;
  std::deque<int32_t> free_list;                 // FIFO: pop front, push back
  std::vector<int32_t> refcount;                 // per page
  std::unordered_map<int32_t, std::vector<int32_t>> tables;
  mutable std::mutex mu;
};

namespace {

int64_t pages_for(int64_t tokens, int32_t page_size) { return (tokens + page_size - 1) / page_size; }

void write_row(const std::vector<int32_t>& pages, int32_t* row, int32_t max_pages) {
  if (!row) return;
  const int32_t n = static_cast<int32_t>(pages.size());
  for (int32_t j = 0; j < max_pages; ++j) row[j] = j < n ? pages[j] : -1;
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
    default: return "PKV_ERR_UNKNOWN";
  }
}

int pkv_abi_version(void) { return 1; }

int pkv_alloc_create(int32_t num_pages, int32_t page_size, const int32_t* free_order,
                     pkv_allocator** out) {
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
  pkv_allocator* a = new (std::nothrow) pkv_allocator();
  if (!a) return PKV_ERR_INVALID_ARG;
  a->num_pages = num_pages;
  a->page_size = page_size;
  a->free_list.assign(order.begin(), order.end());
  a->refcount.assign(static_cast<size_t>(num_pages), 0);
  *out = a;
  return PKV_OK;
}

void pkv_alloc_destroy(pkv_allocator* alloc) { delete alloc; }

int pkv_alloc_reserve_batch(pkv_allocator* a, int32_t B, const int32_t* seqs, const int32_t* n_tokens,
                            int32_t* block_table, int32_t max_pages) {
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
  if (need_total > static_cast<int64_t>(a->free_list.size())) return PKV_ERR_OUT_OF_PAGES;
  // commit: pages leave the free list in batch order
  for (int32_t i = 0; i < B; ++i) {
    const int64_t want = pages_for(n_tokens[i], a->page_size);
    std::vector<int32_t>& tab = a->tables[seqs[i]];
    while (static_cast<int64_t>(tab.size()) < want) {
      const int32_t p = a->free_list.front();
      a->free_list.pop_front();
      a->refcount[p] = 1;
      tab.push_back(p);
    }
  }
  if (block_table) {
    for (int32_t i = 0; i < B; ++i)
      write_row(a->tables[seqs[i]], block_table + static_cast<int64_t>(i) * max_pages, max_pages);
  }
  return PKV_OK;
}

int pkv_alloc_reserve(pkv_allocator* a, int32_t seq, int32_t n_tokens, int32_t* bt_row,
                      int32_t max_pages, int32_t* n_pages) {
  if (!a) return PKV_ERR_INVALID_ARG;
  const int rc = pkv_alloc_reserve_batch(a, 1, &seq, &n_tokens, bt_row, max_pages);
  if (rc == PKV_OK && n_pages) {
    std::lock_guard<std::mutex> lock(a->mu);
    *n_pages = static_cast<int32_t>(a->tables[seq].size());
  }
  return rc;
}

int pkv_alloc_share_prefix(pkv_allocator* a, int32_t seq, const int32_t* pages, int32_t n) {
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
}

int pkv_alloc_free(pkv_allocator* a, int32_t seq) {
  if (!a) return PKV_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(a->mu);
  auto tab = a->tables.find(seq);
  if (tab == a->tables.end()) return PKV_OK;
  for (int32_t p : tab->second) {
    if (--a->refcount[p] == 0) a->free_list.push_back(p);
  }
  a->tables.erase(tab);
  return PKV_OK;
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
                        int32_t N, int32_t exclusive_tail, int32_t* bad_row, int32_t* bad_entry,
                        int32_t* rule) {
  if (B < 0 || max_pages < 0 || P <= 0 || N < 0) return PKV_ERR_INVALID_ARG;
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
  std::vector<int32_t> owners(static_cast<size_t>(N), 0);   // rows referencing each page
  std::vector<int32_t> last_owner(static_cast<size_t>(N), -1);
  std::vector<int32_t> mark(static_cast<size_t>(N), -1);     // row that last saw the page
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = lens[b];
    if (n < 0) return fail(1, b, -1);
    const int64_t used = pages_for(n, P);
    if (used > max_pages) return fail(2, b, -1);
    const int32_t* row = bt + static_cast<int64_t>(b) * max_pages;
    for (int64_t j = 0; j < used; ++j) {
      const int32_t p = row[j];
      if (p < 0 || p >= N) return fail(3, b, static_cast<int32_t>(j));
      if (mark[p] == b) return fail(4, b, static_cast<int32_t>(j));
      mark[p] = b;
      if (last_owner[p] != b) {
        owners[p] += 1;
        last_owner[p] = b;
      }
    }
  }
  if (exclusive_tail) {
    for (int32_t b = 0; b < B; ++b) {
      const int64_t used = pages_for(lens[b], P);
      if (used == 0) continue;
      const int32_t p = bt[static_cast<int64_t>(b) * max_pages + used - 1];
      if (owners[p] > 1) return fail(5, b, static_cast<int32_t>(used - 1));
    }
  }
  return PKV_OK;
}

}  // extern "C"
