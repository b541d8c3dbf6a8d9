"""Reference model of the host page allocator and block-table checks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages ask of KV memory management:
* fixed-size pages allocated independently and reached through a per-sequence
  page table, so a sequence never needs one large contiguous reservation
  (hotelren §3.2, dpshk §4.2, pgsm §3.2);
* allocate on demand and give pages back as soon as a request ends, also when
  it fails (dpshk §4.2);
* requests with a common prefix (a system prompt) share one copy of that
  prefix's KV (dpshk §4.2, pgsm §3.2 and §4.3).

The pages leave the policy open. This model fixes the reading the C++
allocator must reproduce exactly:
* the free list is FIFO: pages are taken from the front in ``free_order``;
  a released page goes to the back;
* ``reserve`` is all-or-nothing: if the free list cannot cover the request
  nothing changes and ``OutOfPages`` is raised;
* shared pages carry a reference count; a page returns to the free list when
  its count reaches zero; ``free`` releases a sequence's pages in table order.
"""

from collections import deque

import numpy as np

from .paged_decode import pages_for_tokens


class OutOfPages(Exception):
    pass


class PageAllocatorModel:
    def __init__(self, num_pages, page_size, free_order=None):
        if num_pages < 0 or page_size <= 0:
            raise ValueError("bad allocator size")
        order = list(range(num_pages)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_pages)):
            raise ValueError("free_order must be a permutation of range(num_pages)")
        self.num_pages = num_pages
        self.page_size = page_size
        self.free_list = deque(order)
        self.refcount = [0] * num_pages
        self.tables = {}

    def free_count(self):
        return len(self.free_list)

    def table(self, seq):
        return list(self.tables.get(seq, []))

    def reserve(self, seq, n_tokens):
        """Make sequence ``seq`` hold at least ``n_tokens`` tokens of pages."""
        if seq < 0 or n_tokens < 0:
            raise ValueError("bad sequence or token count")
        have = self.tables.get(seq, [])
        need = pages_for_tokens(n_tokens, self.page_size) - len(have)
        if need <= 0:
            self.tables.setdefault(seq, have)
            return self.table(seq)
        if need > len(self.free_list):
            raise OutOfPages()
        new = [self.free_list.popleft() for _ in range(need)]
        for p in new:
            self.refcount[p] = 1
        self.tables[seq] = have + new
        return self.table(seq)

    def share_prefix(self, seq, pages):
        """Start ``seq``'s table with already-allocated ``pages`` (count + 1)."""
        if self.tables.get(seq):
            raise ValueError("prefix must be shared into an empty sequence")
        pages = [int(p) for p in pages]
        for p in pages:
            if not (0 <= p < self.num_pages) or self.refcount[p] <= 0:
                raise ValueError("shared page is not allocated")
        if len(set(pages)) != len(pages):
            raise ValueError("duplicate page in shared prefix")
        for p in pages:
            self.refcount[p] += 1
        self.tables[seq] = pages
        return self.table(seq)

    def free(self, seq):
        """Release every page of ``seq``; unknown sequences are a no-op."""
        for p in self.tables.pop(seq, []):
            self.refcount[p] -= 1
            if self.refcount[p] == 0:
                self.free_list.append(p)


def validate_tables(block_table, lens, page_size, num_pages, exclusive_tail=False):
    """Return a list of problems with a block table (empty when valid).

    Checks, on host copies: lengths non-negative and within the row width;
    every entry a token can reach is a page id in ``[0, num_pages)``; no page
    twice in one row; with ``exclusive_tail`` the page holding each sequence's
    last token (the one an append writes) appears in no other row.
    """
    bt = np.asarray(block_table)
    lens = np.asarray(lens)
    problems = []
    owners = {}
    tails = []
    for b in range(bt.shape[0]):
        n = int(lens[b])
        if n < 0:
            problems.append(("negative_length", b, -1))
            continue
        used = pages_for_tokens(n, page_size)
        if used > bt.shape[1]:
            problems.append(("length_exceeds_table", b, -1))
            continue
        seen = set()
        for j in range(used):
            p = int(bt[b, j])
            if not (0 <= p < num_pages):
                problems.append(("page_out_of_range", b, j))
                continue
            if p in seen:
                problems.append(("duplicate_in_row", b, j))
            seen.add(p)
            owners.setdefault(p, set()).add(b)
        if used:
            tails.append((b, used - 1, int(bt[b, used - 1])))
    if exclusive_tail:
        for b, j, p in tails:
            if p in owners and len(owners[p]) > 1:
                problems.append(("shared_tail_page", b, j))
    return problems
