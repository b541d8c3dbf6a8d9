"""Pins for the fp64 oracle: each check ties it to something other than itself.

* closed forms and tables printed on the pages (tests/golden/);
* brute force: pure-Python textbook attention over contiguous K/V on tiny
  inputs, against the oracle reading the same K/V scattered through pages;
* a library routine (torch's scaled-dot-product attention in float64 on CPU);
* exact special cases (one token, zero query, constant values, a spike);
* invariances: physical page permutation and page size;
* the log-sum-exp split identity;
* planted mistakes in the oracle's own source must trip at least one pin.
"""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import paged_decode


def _read_table(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(x) for x in line.split()])
    return rows


# ---------------------------------------------------------------------------
# closed forms printed on the pages
# ---------------------------------------------------------------------------

def test_kv_size_closed_form(golden_dir):
    (layers, heads, dim, seq, nbytes, printed_gb), = _read_table(os.path.join(golden_dir, "kv_size_closed_form.txt"))
    got = oracle.kv_cache_bytes(int(layers), int(heads), int(dim), int(seq), int(nbytes))
    # the printed product: 2 x 32 x 32 x 128 x 4096 x 2
    assert got == 2 * 32 * 32 * 128 * 4096 * 2 == 2_147_483_648
    assert round(got / 1e9, 1) == printed_gb


def test_kv_size_batch_ratios(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "kv_size_batch_table.txt"))
    sizes = [oracle.kv_cache_bytes(32, 32, 128, int(s), 2, batch=int(b)) for b, s, _ in rows]
    printed = [gb for _, _, gb in rows]
    # the printed values scale exactly like the formula (x4 batch, then x2 length)
    for i in range(1, len(rows)):
        assert sizes[i] / sizes[0] == pytest.approx(printed[i] / printed[0], rel=1e-12)
    # the absolute values do not match the formula (page inconsistency, recorded)
    assert sizes[0] == 1_073_741_824
    assert abs(sizes[0] / 1e9 - printed[0]) > 0.5


def test_page_count_table(golden_dir):
    for page_size, pages in _read_table(os.path.join(golden_dir, "page_count_table.txt")):
        page_size, pages = int(page_size), int(pages)
        # every printed row is a 2048-token request
        assert oracle.pages_for_tokens(2048, page_size) == pages
        assert oracle.pages_for_tokens(2048 - page_size + 1, page_size) == pages
        assert oracle.pages_for_tokens(2048 + 1, page_size) == pages + 1


def test_pages_for_tokens_small():
    assert [oracle.pages_for_tokens(n, 16) for n in (0, 1, 15, 16, 17, 32, 33)] == [0, 1, 1, 1, 2, 2, 3]
    with pytest.raises(ValueError):
        oracle.pages_for_tokens(-1, 16)


def test_pool_bytes():
    # one 16 x 128 fp16 tile per (page, head) is 4 KiB; K and V pools
    assert oracle.pool_bytes(1, 1, 16, 128) == 2 * 4096
    assert oracle.pool_bytes(10, 8, 16, 128) == 10 * 8 * 2 * 4096


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

def textbook_attention(q_vec, keys, vals, scale):
    """softmax(scale * q.k_t) weighted sum of v_t, pure Python, fsum."""
    scores = [scale * math.fsum(a * b for a, b in zip(q_vec, k)) for k in keys]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    z = math.fsum(w)
    return [math.fsum(wi * v[d] for wi, v in zip(w, vals)) / z for d in range(len(vals[0]))]


def make_paged_case(rng, B, Hq, Hkv, D, P, lens, spare_pages=3, poison=True):
    """Contiguous fp16 K/V per (sequence, kv head), scattered into a paged pool
    through a random permutation; slots nobody owns hold NaN."""
    max_pages = max(1, max(-(-int(n) // P) for n in lens))
    need = sum(-(-int(n) // P) for n in lens)
    N = need + spare_pages
    perm = rng.permutation(N)
    fill = np.nan if poison else 0.0
    k_pool = np.full(oracle.pool_shape(N, Hkv, P, D), fill, dtype=np.float16)
    v_pool = np.full(oracle.pool_shape(N, Hkv, P, D), fill, dtype=np.float16)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    K = []
    V = []
    cur = 0
    for b in range(B):
        n = int(lens[b])
        kb = rng.standard_normal((Hkv, n, D)).astype(np.float16)
        vb = rng.standard_normal((Hkv, n, D)).astype(np.float16)
        K.append(kb)
        V.append(vb)
        npg = -(-n // P)
        bt[b, :npg] = perm[cur:cur + npg]
        cur += npg
        for t in range(n):
            for kvh in range(Hkv):
                oracle.write_token(k_pool, bt[b, t // P], kvh, t % P, kb[kvh, t], "k")
                oracle.write_token(v_pool, bt[b, t // P], kvh, t % P, vb[kvh, t], "v")
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    return q, k_pool, v_pool, bt, K, V


CASES = [
    # B, Hq, Hkv, D, P, lens
    (1, 1, 1, 32, 16, [1]),
    (2, 2, 2, 32, 16, [5, 3]),
    (3, 4, 2, 32, 16, [17, 1, 40]),
    (2, 4, 1, 64, 16, [33, 16]),
    (3, 4, 4, 32, 32, [1, 15, 40]),
    (2, 2, 1, 64, 32, [9, 70]),
]


@pytest.mark.parametrize("B,Hq,Hkv,D,P,lens", CASES)
def test_brute_force_matches_textbook(B, Hq, Hkv, D, P, lens):
    rng = np.random.default_rng(1000 + B * 7 + P)
    scale = 1.0 / math.sqrt(D)
    q, kp, vp, bt, K, V = make_paged_case(rng, B, Hq, Hkv, D, P, lens)
    got = oracle.decode_attention(q, kp, vp, bt, np.array(lens, np.int32), scale, P)
    g = Hq // Hkv
    s32 = float(np.float32(scale))
    for b in range(B):
        for h in range(Hq):
            ref = textbook_attention(q[b, h].astype(float).tolist(),
                                     K[b][h // g].astype(float).tolist(),
                                     V[b][h // g].astype(float).tolist(), s32)
            np.testing.assert_allclose(got[b, h], ref, rtol=0, atol=1e-12)


def test_library_attention_agrees():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(77)
    B, Hq, Hkv, D, P = 3, 8, 2, 64, 16
    lens = [37, 64, 5]
    q, kp, vp, bt, K, V = make_paged_case(rng, B, Hq, Hkv, D, P, lens)
    scale = 0.125
    got = oracle.decode_attention(q, kp, vp, bt, np.array(lens, np.int32), scale, P)
    for b in range(B):
        qt = torch.from_numpy(q[b].astype(np.float64))[None, :, None, :]      # [1, Hq, 1, D]
        kt = torch.from_numpy(K[b].astype(np.float64))[None]                  # [1, Hkv, n, D]
        vt = torch.from_numpy(V[b].astype(np.float64))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(got[b], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# special cases with exact answers
# ---------------------------------------------------------------------------

def _one_seq(rng, n, D=32, P=16, Hkv=1, Hq=1):
    return make_paged_case(rng, 1, Hq, Hkv, D, P, [n])


def test_single_token_returns_its_value():
    rng = np.random.default_rng(5)
    q, kp, vp, bt, K, V = _one_seq(rng, 1, D=64, P=16, Hkv=2, Hq=4)
    got = oracle.decode_attention(q, kp, vp, bt, np.array([1], np.int32), 0.125, 16)
    for h in range(4):
        assert np.array_equal(got[0, h], V[0][h // 2][0].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(6)
    q, kp, vp, bt, K, V = _one_seq(rng, 29)
    q[:] = 0
    got = oracle.decode_attention(q, kp, vp, bt, np.array([29], np.int32), 0.25, 16)
    np.testing.assert_allclose(got[0, 0], V[0][0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-13)


def test_zero_keys_give_mean_of_values():
    rng = np.random.default_rng(7)
    q, kp, vp, bt, K, V = _one_seq(rng, 23)
    kp[np.isfinite(kp)] = 0
    got = oracle.decode_attention(q, kp, vp, bt, np.array([23], np.int32), 0.25, 16)
    np.testing.assert_allclose(got[0, 0], V[0][0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-13)


def test_constant_values_give_the_constant():
    rng = np.random.default_rng(8)
    q, kp, vp, bt, K, V = _one_seq(rng, 31)
    vp[np.isfinite(vp)] = 1.5
    got = oracle.decode_attention(q, kp, vp, bt, np.array([31], np.int32), 0.25, 16)
    np.testing.assert_allclose(got[0, 0], 1.5, rtol=0, atol=1e-13)


@pytest.mark.parametrize("spike", [0, 3, 15, 16, 30])
def test_spike_key_selects_its_value(spike):
    rng = np.random.default_rng(9)
    n, D, P = 31, 32, 16
    q, kp, vp, bt, K, V = _one_seq(rng, n, D=D, P=P)
    q[0, 0] = np.float16(1.0)
    # every other key zero, the spike a large constant vector
    for t in range(n):
        oracle.write_token(kp, bt[0, t // P], 0, t % P, np.zeros(D, np.float16), "k")
    oracle.write_token(kp, bt[0, spike // P], 0, spike % P, np.full(D, 64.0, np.float16), "k")
    got = oracle.decode_attention(q, kp, vp, bt, np.array([n], np.int32), 1.0, P)
    # the spike's score exceeds the others' by 64 * sum(q) with q >= 0 here
    assert np.array_equal(got[0, 0], V[0][0][spike].astype(np.float64))


def test_empty_sequence_gives_zeros():
    rng = np.random.default_rng(10)
    q, kp, vp, bt, K, V = make_paged_case(rng, 2, 2, 2, 32, 16, [0, 3])
    got = oracle.decode_attention(q, kp, vp, bt, np.array([0, 3], np.int32), 0.5, 16)
    assert np.all(got[0] == 0)
    assert np.all(np.isfinite(got[1]))


# ---------------------------------------------------------------------------
# invariances
# ---------------------------------------------------------------------------

def test_physical_page_permutation_is_invisible():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, D, P = 3, 4, 2, 32, 16
    lens = np.array([13, 49, 8], np.int32)
    q, kp, vp, bt, K, V = make_paged_case(rng, B, Hq, Hkv, D, P, lens)
    base = oracle.decode_attention(q, kp, vp, bt, lens, 0.25, P)
    sigma = rng.permutation(kp.shape[0])          # new page id of old page i
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[sigma] = kp
    vp2[sigma] = vp
    bt2 = np.where(bt >= 0, sigma[np.maximum(bt, 0)], -1).astype(np.int32)
    again = oracle.decode_attention(q, kp2, vp2, bt2, lens, 0.25, P)
    assert np.array_equal(base, again)


def test_page_size_is_invisible():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, D = 2, 4, 2, 32
    lens = [300, 37]
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    K = [rng.standard_normal((Hkv, n, D)).astype(np.float16) for n in lens]
    V = [rng.standard_normal((Hkv, n, D)).astype(np.float16) for n in lens]
    outs = []
    for P in (16, 32, 64, 128):
        npg = [-(-n // P) for n in lens]
        N = sum(npg) + 1
        perm = np.random.default_rng(P).permutation(N)
        kp = np.full(oracle.pool_shape(N, Hkv, P, D), np.nan, np.float16)
        vp = np.full(oracle.pool_shape(N, Hkv, P, D), np.nan, np.float16)
        bt = np.full((B, max(npg)), -1, np.int32)
        cur = 0
        for b, n in enumerate(lens):
            bt[b, :npg[b]] = perm[cur:cur + npg[b]]
            cur += npg[b]
            for t in range(n):
                for kvh in range(Hkv):
                    oracle.write_token(kp, bt[b, t // P], kvh, t % P, K[b][kvh, t], "k")
                    oracle.write_token(vp, bt[b, t // P], kvh, t % P, V[b][kvh, t], "v")
        outs.append(oracle.decode_attention(q, kp, vp, bt, np.array(lens, np.int32), 0.25, P))
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)


@pytest.mark.parametrize("P,D", [(16, 32), (16, 64), (16, 128), (32, 64), (64, 128), (128, 128)])
def test_tile_layouts_are_bijections(P, D):
    t, d = np.meshgrid(np.arange(P), np.arange(D), indexing="ij")
    for f in (oracle.k_tile_offset, oracle.v_tile_offset):
        off = f(t, d, P, D).ravel()
        assert sorted(off.tolist()) == list(range(P * D))


def test_tile_layout_keeps_16_byte_runs():
    # K: 8 consecutive dims of one token are one 16-byte run; V: 4 consecutive
    # tokens (same 4-group) of one dim are one 8-byte run
    P, D = 32, 128
    for tt in range(P):
        for c in range(D // 8):
            off = oracle.k_tile_offset(tt, np.arange(c * 8, c * 8 + 8), P, D)
            assert off[0] % 8 == 0 and np.all(np.diff(off) == 1)
    for g in range(P // 4):
        for dd in range(D):
            off = oracle.v_tile_offset(np.arange(g * 4, g * 4 + 4), dd, P, D)
            assert off[0] % 4 == 0 and np.all(np.diff(off) == 1)


def test_write_then_read_token_roundtrip():
    rng = np.random.default_rng(3)
    pool = np.zeros(oracle.pool_shape(3, 2, 32, 64), np.float16)
    vec = rng.standard_normal(64).astype(np.float16)
    for kind in ("k", "v"):
        oracle.write_token(pool, 2, 1, 17, vec, kind)
        assert np.array_equal(oracle.read_token(pool, 2, 1, 17, kind), vec)
        assert (pool.view(np.uint16) != 0).sum() <= 64 * (2 if kind == "v" else 1)


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------

def test_append_writes_exactly_one_token_per_sequence():
    rng = np.random.default_rng(13)
    B, Hkv, D, P = 3, 2, 32, 16
    lens = np.array([15, 16, 1], np.int32)    # appended positions 15, 16, 1
    q, kp, vp, bt, K, V = make_paged_case(rng, B, 2, Hkv, D, P, lens + 1, poison=False)
    k_new = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    v_new = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    k2, v2 = oracle.kv_append(kp, vp, k_new, v_new, bt, lens, P)
    changed = (k2.view(np.uint16) != kp.view(np.uint16)).sum() + (v2.view(np.uint16) != vp.view(np.uint16)).sum()
    assert changed <= 2 * B * Hkv * D
    assert changed >= 2 * B * Hkv * D - 8      # random fp16 collisions are rare
    for b in range(B):
        keys = oracle.gather_sequence(k2, bt[b], int(lens[b]) + 1, 1, P, "k")
        assert np.array_equal(keys[-1], k_new[b, 1].astype(np.float64))
        assert np.array_equal(keys[:-1], K[b][1][:lens[b]].astype(np.float64))
    assert np.array_equal(kp, kp)  # inputs untouched
    assert not np.shares_memory(k2, kp)


# ---------------------------------------------------------------------------
# split context / log-sum-exp merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("part", [1, 4, 7, 16, 64, 1000])
def test_split_merge_equals_unsplit(part):
    rng = np.random.default_rng(14)
    B, Hq, Hkv, D, P = 3, 4, 2, 32, 16
    lens = np.array([1, 33, 64], np.int32)
    q, kp, vp, bt, K, V = make_paged_case(rng, B, Hq, Hkv, D, P, lens)
    full = oracle.decode_attention(q, kp, vp, bt, lens, 0.3, P)
    parts = oracle.decode_partials(q, kp, vp, bt, lens, 0.3, P, part)
    for b in range(B):
        m, l, o = parts[b]
        assert m.shape[1] == -(-int(lens[b]) // part)
        for h in range(Hq):
            np.testing.assert_allclose(oracle.lse_merge(m[h], l[h], o[h]), full[b, h], rtol=0, atol=1e-12)


def test_lse_merge_closed_form():
    # two partitions, one token each: s = (0, ln 3), v = (1, 5) -> (1*1 + 3*5)/(1+3) = 4
    m = [0.0, math.log(3.0)]
    l = [1.0, 1.0]
    o = [[1.0], [5.0]]
    assert oracle.lse_merge(m, l, o)[0] == pytest.approx(4.0, abs=1e-15)
    assert np.all(oracle.lse_merge([], [], np.zeros((0, 3))) == 0)


# ---------------------------------------------------------------------------
# planted mistakes must trip a pin
# ---------------------------------------------------------------------------

MUTANTS = [
    ("h = kvh * g + i", "h = i * hkv + kvh"),                       # wrong GQA head map
    ("s = s64 * (keys @ qh)", "s = (keys @ qh)"),                  # dropped scale
    ("p = np.exp(s - s.max())", "p = np.exp(s.max() - s)"),        # sign
    ("out[b, h] = (p @ vals) / p.sum()", "out[b, h] = (p @ keys) / p.sum()"),   # K/V swapped
    ("out[b, h] = (p @ vals) / p.sum()", "out[b, h] = (p @ vals) / n"),         # wrong normaliser
    ("[t // page_size]\n", "[t // page_size - (t % page_size == 0) * (t > 0)]\n"),  # page off by one
    ("(t % page_size)[:, None]", "((t + 1) % page_size)[:, None]"),  # slot off by one
    ("return float(np.float32(scale))", "return float(np.float16(scale))"),    # scale precision
    ('keys = gather_sequence(k_pool, block_table[b], n, kvh, page_size, "k")\n            vals',
     'keys = gather_sequence(k_pool, block_table[b], n - 1, kvh, page_size, "k")\n'
     '            keys = np.vstack([keys, keys[-1:]])\n            vals'),  # last token dropped
    ('vals = gather_sequence(v_pool, block_table[b], n, kvh, page_size, "v")\n            for i',
     'vals = gather_sequence(v_pool, block_table[b], n, kvh, page_size, "k")\n            for i'),  # V read as K
]


def _pins_pass(mod):
    """Run a subset of the pins against module ``mod``; False if any fails."""
    try:
        for case in CASES:
            B, Hq, Hkv, D, P, lens = case
            rng = np.random.default_rng(1000 + B * 7 + P)
            scale = 1.0 / math.sqrt(D)
            q, kp, vp, bt, K, V = make_paged_case(rng, B, Hq, Hkv, D, P, lens)
            with np.errstate(all="ignore"):
                got = mod.decode_attention(q, kp, vp, bt, np.array(lens, np.int32), scale, P)
            g = Hq // Hkv
            s32 = float(np.float32(scale))
            for b in range(B):
                for h in range(Hq):
                    ref = textbook_attention(q[b, h].astype(float).tolist(), K[b][h // g].astype(float).tolist(),
                                             V[b][h // g].astype(float).tolist(), s32)
                    if not np.allclose(got[b, h], ref, rtol=0, atol=1e-12):
                        return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("old,new", MUTANTS)
def test_planted_mistake_is_caught(old, new):
    import types
    src = open(paged_decode.__file__).read()
    assert src.count(old) >= 1, old
    mutant = types.ModuleType("oracle_mutant")
    mutant.__dict__["__file__"] = "<mutant>"
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mutant.__dict__)
    assert _pins_pass(paged_decode)
    assert not _pins_pass(mutant), "planted mistake not detected: %r -> %r" % (old, new)


def test_oracle_matches_its_stored_golden(golden_dir):
    import json
    from workloads import workload
    with open(os.path.join(golden_dir, "oracle_tiny_decode.json")) as f:
        ref = json.load(f)
    w = workload(1)
    got = oracle.decode_attention(w.q, w.k_pool, w.v_pool, w.block_table, w.lens(0), w.scale, w.P)
    assert list(got.shape) == ref["shape"]
    np.testing.assert_array_equal(got.ravel(), np.array(ref["values"]))
