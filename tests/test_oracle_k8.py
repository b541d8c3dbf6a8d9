"""Pins for the int8-key oracle (oracle/quant_k8.py).

* exact quantiser cases: zero vectors, a grid the scale divides exactly, ties
  rounded half to even;
* the quantiser's error bound (|k - code * scale| <= scale / 2, the extreme
  value reaching +-127) on random vectors;
* the storage format is a bijection (every code and scale byte has one home)
  and writing then gathering returns each token's dequantised key;
* brute force: textbook attention over the contiguous dequantised keys equals
  the oracle reading them scattered through permuted int8 pages;
* the append changes exactly one token's codes, scale and value per head;
* planted mistakes in the module's source trip at least one of these pins.
"""

import math
import types

import numpy as np
import pytest

import oracle
from oracle import quant_k8


def _fp16(x):
    return np.asarray(x, np.float16)


# ---------------------------------------------------------------------------
# quantiser
# ---------------------------------------------------------------------------

def _check_quantiser(mod):
    # zero vector: scale 0, zero codes
    codes, scale = mod.quantize_k(np.zeros(64, np.float16))
    assert scale == 0 and not codes.any()
    # a grid the scale divides exactly: amax = 127 / 16 gives scale 1 / 16
    vals = np.zeros(64)
    vals[:6] = [127, -64, 1, 0, -127, 3]
    codes, scale = mod.quantize_k(_fp16(vals / 16))
    assert scale == np.float32(1 / 16)
    assert codes[:6].tolist() == [127, -64, 1, 0, -127, 3] and not codes[6:].any()
    # ties: with amax = 127 the scale is exactly 1 and halves round to even
    vals = np.zeros(64)
    vals[:7] = [127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5]
    codes, scale = mod.quantize_k(_fp16(vals))
    assert scale == 1.0
    assert codes[:7].tolist() == [127, 2, 4, -2, 0, 2, 0]
    # error bound on random vectors
    rng = np.random.default_rng(3)
    for trial in range(200):
        k = _fp16(rng.standard_normal(128) * rng.choice([1e-3, 1.0, 30.0]))
        codes, scale = mod.quantize_k(k)
        kf = k.astype(np.float64)
        amax = np.abs(kf).max()
        assert scale == np.float32(np.float32(amax) / np.float32(127))
        assert codes.dtype == np.int8 and np.abs(codes.astype(int)).max() == 127
        assert np.abs(codes.astype(int)).max() <= 127
        # half a step, plus the fp32 roundings of scale, 127 / amax and k * inv (each <= 2^-24
        # relative, on |k| / scale <= 127 steps)
        err = np.abs(kf - codes.astype(np.float64) * float(scale))
        assert err.max() <= float(scale) * (0.5 + 127 * 3 * 2.0 ** -24)


def test_quantiser_pins():
    _check_quantiser(quant_k8)


# ---------------------------------------------------------------------------
# storage format
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("D", [64, 128])
def test_format_is_a_bijection(D):
    u, d = np.meshgrid(np.arange(16), np.arange(D), indexing="ij")
    offs = oracle.k8_code_offset(u, d, D).ravel()
    assert sorted(offs.tolist()) == list(range(16 * D))
    so = oracle.k8_scale_offset(np.arange(16), D)
    assert so.tolist() == list(range(16 * D, 16 * D + 64, 4))
    assert oracle.k8_subblock_bytes(D) == 16 * D + 64
    assert oracle.k8_pool_bytes(10, 8, 32, D) == 10 * 8 * 2 * (16 * D + 64)


def _paged_fp16_pool(rng, N, Hkv, P, D):
    return _fp16(rng.standard_normal(oracle.pool_shape(N, Hkv, P, D)))


@pytest.mark.parametrize("P,D", [(16, 64), (32, 128)])
def test_write_then_gather_returns_dequantised_tokens(P, D):
    rng = np.random.default_rng(P + D)
    N, Hkv = 5, 2
    kp = _paged_fp16_pool(rng, N, Hkv, P, D)
    pool8 = oracle.quantize_k_pool(kp)
    assert pool8.shape == (N, Hkv, P // 16, 16 * D + 64)
    # one sequence over pages in a permuted order
    bt = rng.permutation(N).astype(np.int32)
    L = N * P - 3
    for h in range(Hkv):
        got = oracle.k8_gather_sequence(pool8, bt, L, h, P, D)
        for t in range(L):
            page, off = int(bt[t // P]), t % P
            codes, scale = oracle.quantize_k(oracle.read_token(kp, page, h, off, "k"))
            assert np.array_equal(got[t], codes.astype(np.float64) * float(scale))
            c2, s2 = oracle.k8_read_token(pool8, page, h, off, D)
            assert np.array_equal(c2, codes) and s2 == scale


# ---------------------------------------------------------------------------
# decode over int8 keys
# ---------------------------------------------------------------------------

def _textbook(q, K, V, scale):
    s = [scale * sum(a * b for a, b in zip(q, k)) for k in K]
    m = max(s)
    p = [math.exp(x - m) for x in s]
    z = sum(p)
    return [sum(p[t] * V[t][d] for t in range(len(K))) / z for d in range(len(q))]


def _check_decode(mod, seed=7):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D, P = 2, 4, 2, 64, 16
    N = 7
    lens = np.array([1, 57], np.int32)
    kp = _paged_fp16_pool(rng, N, Hkv, P, D)
    vp = _paged_fp16_pool(rng, N, Hkv, P, D)
    q = _fp16(rng.standard_normal((B, Hq, D)))
    perm = rng.permutation(N).astype(np.int32)
    bt = np.stack([perm[:4], perm[3:7]]).astype(np.int32)
    pool8 = oracle.quantize_k_pool(kp)
    got = mod.decode_attention_k8(q, pool8, vp, bt, lens, 0.125, P)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            K, V = [], []
            for t in range(int(lens[b])):
                page, off = int(bt[b, t // P]), t % P
                codes, scale = oracle.quantize_k(oracle.read_token(kp, page, kvh, off, "k"))
                K.append((codes.astype(np.float64) * float(scale)).tolist())
                V.append(oracle.read_token(vp, page, kvh, off, "v").astype(np.float64).tolist())
            ref = _textbook(q[b, h].astype(np.float64).tolist(), K, V, float(np.float32(0.125)))
            np.testing.assert_allclose(got[b, h], ref, rtol=0, atol=1e-12)
    # with keys that quantise exactly (a grid of the scale) the int8 decode equals fp16 decode
    grid = np.zeros_like(kp)
    for page in range(N):
        for h in range(Hkv):
            for t in range(P):
                vec = rng.integers(-127, 128, size=D) / 64
                vec[0] = 127 / 64                            # every token's amax is 127/64: scale 1/64
                oracle.write_token(grid, page, h, t, _fp16(vec), "k")
    exact = mod.decode_attention_k8(q, oracle.quantize_k_pool(grid), vp, bt, lens, 0.125, P)
    np.testing.assert_allclose(exact, oracle.decode_attention(q, grid, vp, bt, lens, 0.125, P), rtol=0, atol=1e-12)


def test_decode_k8_brute_force_and_exact_grid():
    _check_decode(quant_k8)


def test_append_k8_touches_one_token_per_head():
    rng = np.random.default_rng(11)
    N, Hkv, P, D, B = 6, 2, 16, 128, 3
    kp = _paged_fp16_pool(rng, N, Hkv, P, D)
    vp = _paged_fp16_pool(rng, N, Hkv, P, D)
    pool8 = oracle.quantize_k_pool(kp)
    bt = np.array([[0, 1], [2, 3], [4, 5]], np.int32)
    pos = np.array([0, 17, 31], np.int32)
    kn = _fp16(rng.standard_normal((B, Hkv, D)))
    vn = _fp16(rng.standard_normal((B, Hkv, D)))
    k2, v2 = oracle.kv_append_k8(pool8, vp, kn, vn, bt, pos, P)
    assert np.count_nonzero(k2 != pool8) <= B * Hkv * (D + 4)
    assert np.count_nonzero(v2.view(np.uint16) != vp.view(np.uint16)) <= B * Hkv * D
    for b in range(B):
        page, off = int(bt[b, pos[b] // P]), int(pos[b] % P)
        for h in range(Hkv):
            codes, scale = oracle.k8_read_token(k2, page, h, off, D)
            c0, s0 = oracle.quantize_k(kn[b, h])
            assert np.array_equal(codes, c0) and scale == s0
            assert np.array_equal(oracle.read_token(v2, page, h, off, "v"), vn[b, h])


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

K8_MUTANTS = [
    ("codes = np.rint(k * inv)", "codes = np.trunc(k * inv)"),                        # truncation
    ("inv = np.float32(np.float32(127.0) / amax)", "inv = np.float32(np.float32(128.0) / amax)"),
    ("scale = np.float32(amax / np.float32(127.0))", "scale = np.float32(amax / np.float32(128.0))"),
    ("return codes.view(np.int8).astype(np.float64)", "return codes.astype(np.float64)"),   # unsigned codes
    ("return codes.view(np.int8).astype(np.float64) * scales.astype(np.float64)[:, None]",
     "return codes.view(np.int8).astype(np.float64) * scales.astype(np.float64)[::-1, None]"),   # other tokens' scales
    ("within = t % page_size\n    sub = pool8[pages", "within = (t + 1) % page_size\n    sub = pool8[pages"),  # slot off by one
    ("p = np.exp(s - s.max())", "p = np.exp(s.max() - s)"),                          # sign
    ("s = s64 * (keys @ q[b, h].astype(np.float64))", "s = keys @ q[b, h].astype(np.float64)"),  # dropped scale
]


def _k8_pins_pass(mod):
    try:
        with np.errstate(all="ignore"):
            _check_quantiser(mod)
            _check_decode(mod)
        return True
    except Exception:
        return False


@pytest.mark.parametrize("old,new", K8_MUTANTS)
def test_planted_mistake_is_caught(old, new):
    src = open(quant_k8.__file__).read()
    assert src.count(old) == 1, old
    mutant = types.ModuleType("oracle.quant_k8_mutant")
    mutant.__dict__["__file__"] = "<mutant>"
    mutant.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mutant.__dict__)
    assert _k8_pins_pass(quant_k8)
    assert not _k8_pins_pass(mutant), "planted mistake not detected: %r -> %r" % (old, new)


# ---------------------------------------------------------------------------
# chunks of queries over int8 keys
# ---------------------------------------------------------------------------

def _check_multi_k8(fn, seed=21):
    """Brute force: the causal textbook over the contiguous dequantised keys
    (each token's codes and scale from the quantiser) against the oracle
    reading int8 pages in permuted order; k = 1 is single-query int8 decode."""
    from test_oracle_multi import causal_textbook
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D, P, k = 2, 4, 2, 64, 16, 3
    G = Hq // Hkv
    N = 8
    lens = np.array([k + 2, 41], np.int32)
    kp = _paged_fp16_pool(rng, N, Hkv, P, D)
    vp = _paged_fp16_pool(rng, N, Hkv, P, D)
    pool8 = oracle.quantize_k_pool(kp)
    perm = rng.permutation(N).astype(np.int32)
    bt = np.stack([perm[:3], perm[3:6]]).astype(np.int32)
    q = _fp16(rng.standard_normal((B, k, Hq, D)))
    got = fn(q, pool8, vp, bt, lens, 0.125, P)
    for b in range(B):
        for h in range(Hq):
            kvh = h // G
            K, V = [], []
            for t in range(int(lens[b])):
                page, off = int(bt[b, t // P]), t % P
                codes, sc = oracle.quantize_k(oracle.read_token(kp, page, kvh, off, "k"))
                K.append((codes.astype(np.float64) * float(sc)).tolist())
                V.append(oracle.read_token(vp, page, kvh, off, "v").astype(np.float64).tolist())
            ref = causal_textbook(q[b, :, h].astype(np.float64).tolist(), K, V, float(np.float32(0.125)))
            np.testing.assert_allclose(got[b, :, h], ref, rtol=0, atol=1e-12)
    one = fn(q[:, -1:], pool8, vp, bt, lens, 0.125, P)
    np.testing.assert_array_equal(one[:, 0], oracle.decode_attention_k8(q[:, -1], pool8, vp, bt, lens, 0.125, P))
    short = fn(q, pool8, vp, bt, np.array([k - 1, 41], np.int32), 0.125, P)
    assert np.all(np.isnan(short[0])) and np.all(np.isfinite(short[1]))
    idle = fn(q, pool8, vp, bt, np.array([0, 41], np.int32), 0.125, P)      # an idle batch slot
    assert np.all(idle[0] == 0) and np.array_equal(idle[1], got[1])


def test_multi_k8_brute_force():
    _check_multi_k8(oracle.decode_attention_multi_k8)


@pytest.mark.parametrize("old,new", [
    ("li = np.where(lens64 < k, 0, lens64 - k + i + 1)\n        out[:, i] = decode_attention_k8",
     "li = np.where(lens64 < k, 0, lens64 - k + i)\n        out[:, i] = decode_attention_k8"),
    ("out[:, i] = decode_attention_k8(q[:, i],", "out[:, i] = decode_attention_k8(q[:, k - 1 - i],"),
    ("short = (lens64 < k) & (lens64 != 0)\n    for i in range(k):\n        li = np.where(lens64 < k, 0, lens64 - k + i + 1)\n        out[:, i] = decode_attention_k8",
     "short = (lens64 < 1) & (lens64 != 0)\n    for i in range(k):\n        li = np.where(lens64 < k, 0, lens64 - k + i + 1)\n        out[:, i] = decode_attention_k8"),
    ("short = (lens64 < k) & (lens64 != 0)\n    for i in range(k):\n        li = np.where(lens64 < k, 0, lens64 - k + i + 1)\n        out[:, i] = decode_attention_k8",
     "short = lens64 < k\n    for i in range(k):\n        li = np.where(lens64 < k, 0, lens64 - k + i + 1)\n        out[:, i] = decode_attention_k8"),
])
def test_multi_k8_planted_mistake_is_caught(old, new):
    src = open(quant_k8.__file__).read()
    assert src.count(old) == 1, old
    mutant = types.ModuleType("oracle.quant_k8_mutant")
    mutant.__dict__["__file__"] = "<mutant>"
    mutant.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mutant.__dict__)
    with pytest.raises(AssertionError):
        _check_multi_k8(mutant.decode_attention_multi_k8)


# ---------------------------------------------------------------------------
# sliding window over a ring of int8-key pages
# ---------------------------------------------------------------------------

def _check_window_k8(fn, seed=31):
    """Brute force: tokens written in order into a ring of R pages (later ones
    overwrite earlier ones), keys quantised by the quantiser; the textbook
    attention over the last W tokens' dequantised keys against the oracle;
    then a window covering a ring that never wrapped is int8 decode itself."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D, P, R, W = 2, 4, 2, 64, 16, 3, 33
    G = Hq // Hkv
    N = B * R + 2
    ring = rng.permutation(N)[:B * R].reshape(B, R).astype(np.int32)
    lens = np.array([W - 5, 4 * R * P + 7], np.int32)
    pool8 = np.zeros((N, Hkv, P // 16, oracle.k8_subblock_bytes(D)), np.uint8)
    vp = _paged_fp16_pool(rng, N, Hkv, P, D)
    K, V = [], []
    for b in range(B):
        kb, vb = [], []
        for t in range(int(lens[b])):
            page = int(ring[b, (t // P) % R])
            kt, vt = [], []
            for h in range(Hkv):
                key = _fp16(rng.standard_normal(D))
                codes, sc = oracle.quantize_k(key)
                oracle.k8_write_token(pool8, page, h, t % P, codes, sc, D)
                val = _fp16(rng.standard_normal(D))
                oracle.write_token(vp, page, h, t % P, val, "v")
                kt.append(codes.astype(np.float64) * float(sc))
                vt.append(val.astype(np.float64))
            kb.append(kt)
            vb.append(vt)
        K.append(kb)
        V.append(vb)
    q = _fp16(rng.standard_normal((B, Hq, D)))
    got = fn(q, pool8, vp, ring, lens, W, 0.125, P)
    for b in range(B):
        lo = max(0, int(lens[b]) - W)
        for h in range(Hq):
            kvh = h // G
            keys = [K[b][t][kvh].tolist() for t in range(lo, int(lens[b]))]
            vals = [V[b][t][kvh].tolist() for t in range(lo, int(lens[b]))]
            ref = _textbook(q[b, h].astype(np.float64).tolist(), keys, vals, float(np.float32(0.125)))
            np.testing.assert_allclose(got[b, h], ref, rtol=0, atol=1e-12)
    # a ring that never wrapped, the window covering everything: int8 decode over the ring as a table
    short = np.array([20, (R - 1) * P + 1], np.int32)
    whole = fn(q, pool8, vp, ring, short, (R - 1) * P + 1, 0.125, P)
    np.testing.assert_array_equal(whole, oracle.decode_attention_k8(q, pool8, vp, ring, short, 0.125, P))


def test_window_k8_brute_force():
    _check_window_k8(oracle.decode_attention_window_k8)


@pytest.mark.parametrize("old,new", [
    ("t = np.arange(max(0, length - window), length)\n        pages = ring[b][(t // page_size) % r]\n        within",
     "t = np.arange(max(0, length - window + 1), length)\n        pages = ring[b][(t // page_size) % r]\n        within"),
    ("pages = ring[b][(t // page_size) % r]\n        within", "pages = ring[b][(t // page_size) % (r - 1)]\n        within"),
    ("codes.view(np.int8).astype(np.float64) * scales.astype(np.float64)[:, None]\n            vals",
     "codes.astype(np.float64) * scales.astype(np.float64)[:, None]\n            vals"),
])
def test_window_k8_planted_mistake_is_caught(old, new):
    src = open(quant_k8.__file__).read()
    assert src.count(old) == 1, old
    mutant = types.ModuleType("oracle.quant_k8_mutant")
    mutant.__dict__["__file__"] = "<mutant>"
    mutant.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mutant.__dict__)
    with pytest.raises((AssertionError, IndexError)):
        _check_window_k8(mutant.decode_attention_window_k8)


def test_window_chunks_k8_are_per_query_window_decodes():
    """Chunks over an int8-key ring: query i equals the int8 window decode of
    its own prefix (checked against the pinned window oracle), short rows NaN."""
    rng = np.random.default_rng(44)
    B, Hq, Hkv, D, P, R, W, k = 2, 4, 2, 64, 16, 4, 40, 3
    N = B * R + 2
    ring = rng.permutation(N)[:B * R].reshape(B, R).astype(np.int32)
    kp = _paged_fp16_pool(rng, N, Hkv, P, D)
    vp = _paged_fp16_pool(rng, N, Hkv, P, D)
    pool8 = oracle.quantize_k_pool(kp)
    lens = np.array([k + 1, 5 * R * P + 3], np.int32)
    q = _fp16(rng.standard_normal((B, k, Hq, D)))
    got = oracle.decode_attention_window_multi_k8(q, pool8, vp, ring, lens, W, 0.125, P)
    for i in range(k):
        li = lens - k + i + 1
        np.testing.assert_array_equal(got[:, i], oracle.decode_attention_window_k8(q[:, i], pool8, vp, ring, li, W,
                                                                                   0.125, P))
    short = oracle.decode_attention_window_multi_k8(q, pool8, vp, ring, np.array([k - 1, 50], np.int32), W, 0.125, P)
    assert np.all(np.isnan(short[0])) and np.all(np.isfinite(short[1]))
