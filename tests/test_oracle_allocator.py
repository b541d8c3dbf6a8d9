"""Pins for the allocator reference model and the block-table checker.

The model's policy (FIFO free list, all-or-nothing reserve, reference-counted
shared prefixes) is a reading of the pages; these tests pin it to invariants
that any correct page allocator must keep, to the page-count table the pages
print, and to a brute-force re-count of ownership after random operation
sequences.
"""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import PageAllocatorModel, OutOfPages, validate_tables


def test_reserve_takes_pages_in_free_order():
    a = PageAllocatorModel(8, 16, free_order=[5, 2, 7, 0, 1, 3, 4, 6])
    assert a.reserve(0, 33) == [5, 2, 7]           # ceil(33/16) = 3 pages
    assert a.reserve(1, 16) == [0]
    assert a.reserve(0, 48) == [5, 2, 7]           # already enough
    assert a.reserve(0, 49) == [5, 2, 7, 1]
    assert a.free_count() == 3


def test_page_count_table_via_reserve():
    # pgsm §4.1 table: a 2048-token request needs 128/64/32/16 pages
    for P, pages in ((16, 128), (32, 64), (64, 32), (128, 16)):
        a = PageAllocatorModel(200, P)
        assert len(a.reserve(0, 2048)) == pages


def test_reserve_is_all_or_nothing():
    a = PageAllocatorModel(4, 16)
    a.reserve(0, 40)                                 # 3 pages
    before = (list(a.free_list), dict(a.tables), list(a.refcount))
    with pytest.raises(OutOfPages):
        a.reserve(1, 40)
    with pytest.raises(OutOfPages):
        a.reserve(0, 80)                             # needs 2 more, 1 free
    assert (list(a.free_list), dict(a.tables), list(a.refcount)) == before


def test_free_returns_pages_to_the_back():
    a = PageAllocatorModel(4, 16, free_order=[3, 2, 1, 0])
    a.reserve(0, 32)                                 # [3, 2]
    a.reserve(1, 16)                                 # [1]
    a.free(0)
    assert list(a.free_list) == [0, 3, 2]
    a.free(0)                                        # unknown: no-op
    assert a.reserve(2, 48) == [0, 3, 2]


def test_shared_prefix_refcounts():
    a = PageAllocatorModel(10, 16)
    prefix = a.reserve(100, 32)                      # owner of the prefix: pages [0, 1]
    a.share_prefix(0, prefix)
    a.share_prefix(1, prefix)
    assert a.reserve(0, 40) == [0, 1, 2]
    assert a.reserve(1, 33) == [0, 1, 3]
    a.free(100)
    a.free(0)
    assert 0 not in a.free_list and 1 not in a.free_list
    a.free(1)
    assert set(a.free_list) == set(range(10))
    with pytest.raises(ValueError):
        a.share_prefix(5, [9])                        # not allocated


OPS = st.lists(
    st.tuples(st.sampled_from(["reserve", "free", "share"]), st.integers(0, 5), st.integers(0, 120)),
    max_size=60)


@settings(max_examples=200, deadline=None)
@given(OPS, st.integers(1, 40), st.sampled_from([1, 4, 16]))
def test_random_operation_sequences_keep_invariants(ops, n_pages, P):
    a = PageAllocatorModel(n_pages, P, free_order=list(np.random.default_rng(n_pages).permutation(n_pages)))
    for kind, seq, n in ops:
        if kind == "reserve":
            before = (list(a.free_list), {k: list(v) for k, v in a.tables.items()})
            try:
                row = a.reserve(seq, n)
                assert len(row) >= oracle.pages_for_tokens(n, P)
            except OutOfPages:
                assert (list(a.free_list), {k: list(v) for k, v in a.tables.items()}) == before
        elif kind == "free":
            a.free(seq)
        else:
            donor = a.tables.get((seq + 1) % 6)
            if donor and not a.tables.get(seq):
                a.share_prefix(seq, donor[: max(1, len(donor) // 2)])
        # brute-force recount of ownership
        count = [0] * n_pages
        for pages in a.tables.values():
            assert len(set(pages)) == len(pages)
            for p in pages:
                count[p] += 1
        assert count == a.refcount
        assert sorted(list(a.free_list) + [p for p in range(n_pages) if count[p] > 0]) == list(range(n_pages))
        assert all(count[p] == 0 for p in a.free_list)


def test_validate_tables_detects_problems():
    bt = np.array([[3, 1, -1], [0, 2, -1]], np.int32)
    assert validate_tables(bt, [20, 17], 16, 4) == []
    assert validate_tables(bt, [20, 40], 16, 4) == [("page_out_of_range", 1, 2)]
    assert validate_tables(bt, [20, 49], 16, 4) == [("length_exceeds_table", 1, -1)]
    assert validate_tables(bt, [-1, 3], 16, 4) == [("negative_length", 0, -1)]
    assert validate_tables(np.array([[3, 3]], np.int32), [20], 16, 4) == [("duplicate_in_row", 0, 1)]
    assert validate_tables(np.array([[9]], np.int32), [1], 16, 4) == [("page_out_of_range", 0, 0)]
    shared = np.array([[0, 1], [0, 2]], np.int32)
    assert validate_tables(shared, [20, 20], 16, 3, exclusive_tail=True) == []
    assert validate_tables(shared, [16, 20], 16, 3, exclusive_tail=True) == [("shared_tail_page", 0, 0)]
    assert validate_tables(shared, [16, 20], 16, 3) == []
    # shared prefix (dpshk §4.2): every attended row holds it in the same pages; idle rows hold anything
    pre = np.array([[-1, -1, -1], [0, 1, 2], [0, 1, 3], [0, 4, 5]], np.int32)
    assert validate_tables(pre[:3], [0, 40, 40], 16, 6, prefix_tokens=32) == []
    assert validate_tables(pre, [0, 40, 40, 40], 16, 6, prefix_tokens=32) == [("prefix_differs", 3, 1)]
    assert validate_tables(pre[:3], [0, 40, 20], 16, 6, prefix_tokens=32) == [("shorter_than_prefix", 2, -1)]
    # rings (hotelren §3.2): the entries the window reaches, in token order
    ring = np.array([[0, 1, 2]], np.int32)
    assert validate_tables(ring, [100], 16, 3, window=33) == []
    assert validate_tables(np.array([[0, 1, 9]], np.int32), [100], 16, 3, window=33) == [("page_out_of_range", 0, 2)]
    assert validate_tables(np.array([[9, 1, 2]], np.int32), [96], 16, 3, window=17) == []
    assert validate_tables(np.array([[1, 1, 2]], np.int32), [100], 16, 3, window=33) == [("duplicate_in_row", 0, 0)]


# ---------------------------------------------------------------------------
# prefix cache and copy on write
# ---------------------------------------------------------------------------

def _state(a):
    return (list(a.free_list), {k: list(v) for k, v in a.tables.items()}, list(a.refcount),
            {k: (list(v[0]), v[1], v[2]) for k, v in a.cache.items()}, a.clock)


def _recount(a):
    """Brute-force ownership: tables plus cache entries; free pages own nothing."""
    count = [0] * a.num_pages
    for pages in a.tables.values():
        assert len(set(pages)) == len(pages)
        for p in pages:
            count[p] += 1
    for pages, _, _ in a.cache.values():
        for p in pages:
            count[p] += 1
    assert count == a.refcount
    assert sorted(list(a.free_list) + [p for p in range(a.num_pages) if count[p] > 0]) == list(range(a.num_pages))


def test_cached_prefix_outlives_its_sequence():
    a = PageAllocatorModel(10, 16)
    a.reserve(0, 40)                                    # pages 0, 1, 2
    assert a.cache_insert(7, 0, 40) == [0, 1, 2]
    a.free(0)
    assert a.free_count() == 7 and a.refcount[:3] == [1, 1, 1]     # the cache holds them
    pages, n = a.cache_lookup(7)
    assert (pages, n) == ([0, 1, 2], 40)
    a.share_prefix(1, pages)
    assert a.refcount[:3] == [2, 2, 2]
    assert a.cache_lookup(99) is None
    a.cache_evict(7)
    a.free(1)
    assert a.free_count() == 10
    _recount(a)


def test_copy_on_write_of_a_shared_partial_page():
    P = 16
    a = PageAllocatorModel(10, P)
    a.reserve(0, 40)                                    # 2.5 pages: the third page is partly filled
    a.share_prefix(1, a.table(0))                       # sequence 1 starts from the same 40 tokens
    a.share_prefix(2, a.table(0)[:2])                   # sequence 2 shares only the two full pages
    # sequences 0 and 1 both append at token 40, inside the shared third page: the first gets a
    # copy, after which the second is the page's only owner and keeps it
    copies = a.prepare_append([0, 1, 2], [40, 40, 32])
    assert copies == [(2, 3)]
    assert a.table(0) == [0, 1, 3] and a.table(1) == [0, 1, 2] and a.table(2) == [0, 1, 4]
    assert a.refcount[2] == 1 and a.refcount[3] == 1 and a.refcount[:2] == [3, 3]
    # the next token of each lands in its own page now: no copies
    assert a.prepare_append([0, 1], [41, 41]) == []
    # a token beyond the table grows it as reserve does
    assert a.prepare_append([2], [48]) == [] and a.table(2) == [0, 1, 4, 5]
    # a shared full page is copied too when written (here: rewrite token 5 of sequence 2)
    assert a.prepare_append([2], [5]) == [(0, 6)] and a.table(2) == [6, 1, 4, 5]
    _recount(a)


def test_prepare_append_is_all_or_nothing_and_evicts_lru_first():
    P = 16
    a = PageAllocatorModel(6, P)
    a.reserve(0, 16)
    a.cache_insert(1, 0, 16)                            # page 0 in cache entry 1 (oldest)
    a.reserve(1, 16)
    a.cache_insert(2, 1, 16)                            # page 1 in cache entry 2
    a.free(0)
    a.free(1)                                           # pages 0 and 1 now held by the cache only
    a.reserve(2, 64)                                    # pages 2..5: free list empty
    assert a.free_count() == 0
    a.cache_lookup(1)                                   # entry 1 becomes the most recent
    before = _state(a)
    with pytest.raises(OutOfPages):
        a.prepare_append([3], [48])                     # needs 4 pages, eviction frees only 2
    assert _state(a) == before
    a.prepare_append([3], [0])                          # 1 page: evicts entry 2 (least recent) only
    assert 2 not in a.cache and 1 in a.cache
    assert a.table(3) == [1]
    _recount(a)


CACHE_OPS = st.lists(
    st.tuples(st.sampled_from(["reserve", "free", "share", "insert", "lookup", "evict", "append"]),
              st.integers(0, 5), st.integers(0, 120)),
    max_size=60)


@settings(max_examples=200, deadline=None)
@given(CACHE_OPS, st.integers(1, 40), st.sampled_from([1, 4, 16]))
def test_random_cache_and_append_sequences_keep_invariants(ops, n_pages, P):
    a = PageAllocatorModel(n_pages, P, free_order=list(np.random.default_rng(n_pages).permutation(n_pages)))
    for kind, seq, n in ops:
        before = _state(a)
        try:
            if kind == "reserve":
                a.reserve(seq, n)
            elif kind == "free":
                a.free(seq)
            elif kind == "share":
                entry = a.cache_lookup(seq % 3)
                if entry and not a.tables.get(seq):
                    a.share_prefix(seq, entry[0])
            elif kind == "insert":
                have = len(a.tables.get(seq, []))
                if have and n:
                    a.cache_insert(seq % 3, seq, min(n, have * P))
            elif kind == "lookup":
                a.cache_lookup(seq % 3)
            elif kind == "evict":
                a.cache_evict(seq % 3)
            else:
                copies = a.prepare_append([seq, (seq + 1) % 6], [n, n // 2])
                for src, dst in copies:
                    assert a.refcount[dst] == 1 and src != dst
        except OutOfPages:
            assert _state(a) == before
        _recount(a)
