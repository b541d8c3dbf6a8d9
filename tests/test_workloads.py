"""The seeded input recipe: determinism and the structure each workload promises."""

import numpy as np
import pytest

import oracle
from workloads import workload
from _helpers import poison_unused


def test_deterministic():
    a, b = workload(2, batch=3), workload(2, batch=3)
    for name in ("q", "k_pool", "v_pool", "block_table", "context", "k_new", "v_new"):
        assert np.array_equal(getattr(a, name).view(np.uint8), getattr(b, name).view(np.uint8))


def test_tiny_workload_shape():
    w = workload(1)
    assert (w.B, w.Hq, w.Hkv, w.D, w.P, w.N) == (1, 4, 4, 64, 16, 64)
    assert w.block_table.shape == (1, 16) and len(set(w.block_table[0].tolist())) == 16
    assert w.steps == 0 and list(w.lens(0)) == [256]
    assert w.scale == 0.125


@pytest.mark.parametrize("number", [2, 3, 5])
def test_pool_sized_to_demand_and_pages_distinct(number):
    w = workload(number, batch=4)
    rows = []
    for b in range(w.B):
        need = oracle.pages_for_tokens(int(w.context[b]) + w.steps, w.P)
        row = w.block_table[b, :need]
        assert np.all(row >= 0) and np.all(w.block_table[b, need:] == -1)
        rows.append(row)
    private = np.concatenate([r[w.shared_prefix_pages:] for r in rows])
    assert len(set(private.tolist())) == len(private)
    assert w.N == w.shared_prefix_pages + len(private)


def test_prefix_workload_shares_first_128_pages():
    w = workload(3, batch=6)
    assert w.shared_prefix_pages == 128
    for b in range(1, w.B):
        assert np.array_equal(w.block_table[b, :128], w.block_table[0, :128])
    private = w.context - 2048
    assert private.min() >= 128 and private.max() <= 8192
    # appends land after the prefix: never in a shared page
    assert np.all(w.pos(0) // 16 >= 128)


def test_length_ranges():
    w2 = workload(2)
    assert w2.context.min() >= 200 and w2.context.max() <= 4096
    w5 = workload(5, page_size=64, batch=8)
    assert w5.context.min() >= 200 and w5.context.max() <= 4000 and w5.steps == 64 and w5.P == 64


def test_poison_marks_only_unused_slots():
    w = workload(2, batch=2)
    lens = w.lens(0)
    k, v = poison_unused(w, lens)
    for b in range(w.B):
        keys = oracle.gather_sequence(k, w.block_table[b], int(lens[b]), 0, w.P, "k")
        vals = oracle.gather_sequence(v, w.block_table[b], int(lens[b]), 0, w.P, "v")
        assert np.all(np.isfinite(vals))
        assert np.all(np.isfinite(keys))
    assert np.isnan(k.astype(np.float32)).sum() == w.N * w.P * w.Hkv * w.D - sum(int(n) for n in lens) * w.Hkv * w.D


def test_sliding_window_workload_ring():
    w = workload(6, batch=4)
    assert (w.Hq, w.Hkv, w.D, w.P, w.window) == (32, 8, 128, 16, 4096)
    R = w.block_table.shape[1]
    # a 4096-token window that starts inside a page touches 257 pages
    assert R == 257 and (R - 1) * w.P + 1 >= w.window
    assert w.N == w.B * R and sorted(w.block_table.ravel().tolist()) == list(range(w.N))
    assert w.context.min() >= w.window and w.context.max() <= 8 * w.window and w.steps == 1
    assert w.k_pool.shape == (w.N, 8, 1, 16 * 128)
