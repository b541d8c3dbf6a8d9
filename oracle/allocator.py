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

The prefix-cache lifecycle (the pages ask for shared prefixes, dpshk §4.2 and
pgsm §3.2, and for reuse of a prompt's KV across requests, pgsm §4.3; the
mechanics below are this library's reading):
* ``cache_insert(key, seq, n_tokens)`` keeps the pages holding the first
  ``n_tokens`` tokens of ``seq`` under ``key`` (a caller-chosen identifier of
  the prompt, e.g. a hash of its tokens); the cache holds one reference on each
  page, so the pages outlive the sequence; inserting an existing key only
  refreshes it;
* ``cache_lookup(key)`` returns ``(pages, n_tokens)`` (or None) and refreshes
  the entry; a new sequence starts from them with ``share_prefix``;
* entries are ordered by last use (insert or lookup, a counter per event);
  when a reservation needs more pages than are free, the least recently used
  entries are dropped (their references released) one at a time until the
  request fits -- but only if dropping all of them would make it fit;
  otherwise nothing changes and ``OutOfPages`` is raised;
* ``prepare_append(seqs, pos)`` readies a batch for writing token ``pos[i]`` of
  sequence ``seqs[i]``: the table grows to hold it (as ``reserve``), and if the
  page it lands in is shared (count > 1) the sequence gets a private copy:
  a new page replaces it in the table, the old page's count drops by one, and
  the pair (old, new) is returned so the caller copies the page's contents on
  the device before writing (copy on write). The whole batch is planned first
  and committed only if the free list (after evictions) covers it.
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
        self.cache = {}          # key -> [pages, n_tokens, last_use]
        self.clock = 0

    def free_count(self):
        return len(self.free_list)

    def table(self, seq):
        return list(self.tables.get(seq, []))

    # -- prefix cache ---------------------------------------------------------

    def _tick(self):
        self.clock += 1
        return self.clock

    def cache_insert(self, key, seq, n_tokens):
        """Keep the pages of ``seq``'s first ``n_tokens`` tokens under ``key``."""
        have = self.tables.get(seq, [])
        n_pages = pages_for_tokens(n_tokens, self.page_size)
        if n_tokens <= 0 or n_pages > len(have):
            raise ValueError("the sequence does not hold that many tokens")
        if key in self.cache:
            self.cache[key][2] = self._tick()
            return list(self.cache[key][0])
        pages = list(have[:n_pages])
        for p in pages:
            self.refcount[p] += 1
        self.cache[key] = [pages, int(n_tokens), self._tick()]
        return list(pages)

    def cache_lookup(self, key):
        """``(pages, n_tokens)`` kept under ``key`` (refreshed), or None."""
        entry = self.cache.get(key)
        if entry is None:
            return None
        entry[2] = self._tick()
        return list(entry[0]), entry[1]

    def _release(self, pages):
        for p in pages:
            self.refcount[p] -= 1
            if self.refcount[p] == 0:
                self.free_list.append(p)

    def cache_evict(self, key):
        """Drop ``key``'s entry (its references); unknown keys are a no-op."""
        entry = self.cache.pop(key, None)
        if entry is not None:
            self._release(entry[0])

    def _make_room(self, need):
        """Evict least recently used entries until ``need`` pages are free, if
        evicting all of them would do; else change nothing and raise."""
        if need <= len(self.free_list):
            return
        # pages that evicting every entry would free: counts held only by the cache
        held = {}
        for pages, _, _ in self.cache.values():
            for p in pages:
                held[p] = held.get(p, 0) + 1
        freeable = sum(1 for p, c in held.items() if self.refcount[p] == c)
        if need > len(self.free_list) + freeable:
            raise OutOfPages()
        for key in sorted(self.cache, key=lambda k: self.cache[k][2]):
            if need <= len(self.free_list):
                break
            self.cache_evict(key)

    # -- pages of sequences ---------------------------------------------------

    def reserve(self, seq, n_tokens):
        """Make sequence ``seq`` hold at least ``n_tokens`` tokens of pages."""
        if seq < 0 or n_tokens < 0:
            raise ValueError("bad sequence or token count")
        have = self.tables.get(seq, [])
        need = pages_for_tokens(n_tokens, self.page_size) - len(have)
        if need <= 0:
            self.tables.setdefault(seq, have)
            return self.table(seq)
        self._make_room(need)
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
        self._release(self.tables.pop(seq, []))

    def prepare_append(self, seqs, pos):
        """Ready every ``seqs[i]`` to have token ``pos[i]`` written (see the
        module notes); returns the list of ``(src, dst)`` page copies."""
        seqs = [int(x) for x in seqs]
        pos = [int(x) for x in pos]
        if len(set(seqs)) != len(seqs) or any(s < 0 for s in seqs) or any(t < 0 for t in pos):
            raise ValueError("bad batch")
        need = 0
        for s, t in zip(seqs, pos):
            have = self.tables.get(s, [])
            j = t // self.page_size
            grow = max(0, j + 1 - len(have))
            shared = j < len(have) and self.refcount[have[j]] > 1
            need += grow + (1 if shared else 0)
        self._make_room(need)
        copies = []
        for s, t in zip(seqs, pos):
            self.reserve(s, t + 1)
            tab = self.tables[s]
            j = t // self.page_size
            old = tab[j]
            if self.refcount[old] > 1:
                new = self.free_list.popleft()
                self.refcount[new] = 1
                self.refcount[old] -= 1
                tab[j] = new
                copies.append((old, new))
        return copies


def _reached_entries(n, page_size, width, window):
    """Block-table entries the tokens of a length-``n`` row reach, in token
    order: logical pages ``0 .. ceil(n / P) - 1``; under a sliding window over a
    ring of ``width`` pages, the ring entries ``j % width`` of the logical pages
    holding tokens ``max(0, n - window) .. n - 1`` (hotelren §3.2's ring of
    preallocated pages, expressed through the page table)."""
    if n <= 0:
        return []
    if window:
        lo = max(0, n - window)
        return [j % width for j in range(lo // page_size, (n - 1) // page_size + 1)]
    return list(range(pages_for_tokens(n, page_size)))


def validate_tables(block_table, lens, page_size, num_pages, exclusive_tail=False, prefix_tokens=0, window=0):
    """Return a list of problems with a block table (empty when valid).

    Checks, on host copies: lengths non-negative and (without a window) within
    the row width; every entry a token can reach is a page id in
    ``[0, num_pages)``; no page twice among a row's reached entries; with
    ``exclusive_tail`` the page holding each sequence's last token (the one an
    append writes) appears in no other row; with ``prefix_tokens`` every
    attended row (length > 0) is at least that long and holds the shared
    prefix in the same pages as the first attended row (dpshk §4.2: one copy
    of a shared prompt serves every request that starts with it). ``window``
    reads the rows as rings (``_reached_entries``); it must fit the ring.
    """
    bt = np.asarray(block_table)
    lens = np.asarray(lens)
    width = bt.shape[1]
    if window and prefix_tokens:
        raise ValueError("a window leaves no shared prefix")
    if prefix_tokens % page_size:
        raise ValueError("the shared prefix is whole pages")
    if window and window > (width - 1) * page_size + 1:
        raise ValueError("the window must fit in the ring")
    problems = []
    owners = {}
    tails = []
    for b in range(bt.shape[0]):
        n = int(lens[b])
        if n < 0:
            problems.append(("negative_length", b, -1))
            continue
        if not window and pages_for_tokens(n, page_size) > width:
            problems.append(("length_exceeds_table", b, -1))
            continue
        seen = set()
        entries = _reached_entries(n, page_size, width, window)
        for j in entries:
            p = int(bt[b, j])
            if not (0 <= p < num_pages):
                problems.append(("page_out_of_range", b, j))
                continue
            if p in seen:
                problems.append(("duplicate_in_row", b, j))
            seen.add(p)
            owners.setdefault(p, set()).add(b)
        if entries:
            tails.append((b, entries[-1], int(bt[b, entries[-1]])))
    if exclusive_tail:
        for b, j, p in tails:
            if p in owners and len(owners[p]) > 1:
                problems.append(("shared_tail_page", b, j))
    if prefix_tokens:
        first = None
        for b in range(bt.shape[0]):
            n = int(lens[b])
            if n == 0:
                continue
            if n < prefix_tokens:
                problems.append(("shorter_than_prefix", b, -1))
                continue
            if first is None:
                first = b
                continue
            for j in range(prefix_tokens // page_size):
                if int(bt[b, j]) != int(bt[first, j]):
                    problems.append(("prefix_differs", b, j))
                    break
    return problems
