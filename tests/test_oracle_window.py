"""Pins for the sliding-window (ring of pages) oracle.

* brute force: textbook attention over the contiguous last W tokens, against
  the oracle reading them through a ring of permuted pages that has wrapped
  (the overwritten slots hold other tokens);
* a window covering the whole sequence in a ring that never wrapped is plain
  decode attention over the same pages;
* tokens outside the window do not matter (rewriting them changes nothing).
"""

import math

import numpy as np
import pytest

import oracle
from test_oracle_pins import textbook_attention


def _ring_case(rng, B, Hkv, D, P, R, lens, extra_pages=2):
    """Contiguous K/V of each sequence written into a ring of R pages (token t
    in page ring[b][(t // P) % R]): later tokens overwrite earlier ones."""
    N = B * R + extra_pages
    perm = rng.permutation(N)
    ring = perm[:B * R].reshape(B, R).astype(np.int32)
    kp = np.full(oracle.pool_shape(N, Hkv, P, D), np.nan, np.float16)
    vp = np.full(oracle.pool_shape(N, Hkv, P, D), np.nan, np.float16)
    K, V = [], []
    for b in range(B):
        n = int(lens[b])
        kb = rng.standard_normal((Hkv, n, D)).astype(np.float16)
        vb = rng.standard_normal((Hkv, n, D)).astype(np.float16)
        K.append(kb)
        V.append(vb)
        for t in range(n):
            page = int(ring[b, (t // P) % R])
            for h in range(Hkv):
                oracle.write_token(kp, page, h, t % P, kb[h, t], "k")
                oracle.write_token(vp, page, h, t % P, vb[h, t], "v")
    return ring, kp, vp, K, V


@pytest.mark.parametrize("P,R,W", [(16, 3, 33), (16, 4, 49), (32, 2, 20), (16, 5, 64)])
def test_window_brute_force_over_a_wrapped_ring(P, R, W):
    rng = np.random.default_rng(P * R + W)
    B, Hkv, G, D = 3, 2, 2, 32
    Hq = Hkv * G
    lens = np.array([W - 7, R * P * 3 + 5, W + 17], np.int32)       # short, wrapped three times, just past W
    ring, kp, vp, K, V = _ring_case(rng, B, Hkv, D, P, R, lens)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    got = oracle.decode_attention_window(q, kp, vp, ring, lens, W, 0.2, P)
    s32 = float(np.float32(0.2))
    for b in range(B):
        lo = max(0, int(lens[b]) - W)
        for h in range(Hq):
            kvh = h // G
            ref = textbook_attention(q[b, h].astype(float).tolist(), K[b][kvh, lo:].astype(float).tolist(),
                                     V[b][kvh, lo:].astype(float).tolist(), s32)
            np.testing.assert_allclose(got[b, h], ref, rtol=0, atol=1e-12)


def test_unwrapped_full_window_is_decode():
    rng = np.random.default_rng(2)
    B, Hkv, G, D, P, R = 2, 2, 4, 32, 16, 6
    lens = np.array([37, 80], np.int32)                            # at most 5 pages: the ring never wraps
    ring, kp, vp, K, V = _ring_case(rng, B, Hkv, D, P, R, lens)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float16)
    got = oracle.decode_attention_window(q, kp, vp, ring, lens, (R - 1) * P + 1, 0.3, P)
    assert np.array_equal(got, oracle.decode_attention(q, kp, vp, ring, lens, 0.3, P))


def test_tokens_outside_the_window_do_not_matter():
    rng = np.random.default_rng(4)
    B, Hkv, G, D, P, R, W = 2, 2, 2, 32, 16, 4, 40
    lens = np.array([70, 100], np.int32)
    ring, kp, vp, K, V = _ring_case(rng, B, Hkv, D, P, R, lens)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float16)
    base = oracle.decode_attention_window(q, kp, vp, ring, lens, W, 0.3, P)
    # rewrite every slot holding a token older than the window (those still in the ring)
    kp2, vp2 = kp.copy(), vp.copy()
    for b in range(B):
        n = int(lens[b])
        for t in range(max(0, n - R * P), n - W):
            page = int(ring[b, (t // P) % R])
            for h in range(Hkv):
                oracle.write_token(kp2, page, h, t % P, np.full(D, 9.0, np.float16), "k")
                oracle.write_token(vp2, page, h, t % P, np.full(D, -9.0, np.float16), "v")
    assert np.array_equal(oracle.decode_attention_window(q, kp2, vp2, ring, lens, W, 0.3, P), base)
    with pytest.raises(ValueError):
        oracle.decode_attention_window(q, kp, vp, ring, lens, (R - 1) * P + 2, 0.3, P)


def _window_causal_textbook(Q, K, V, scale, W):
    """Q [k][D], K/V [L][D] contiguous: query i sits at p = L - k + i and sees
    keys max(0, p + 1 - W) .. p only."""
    k, L = len(Q), len(K)
    out = []
    for i in range(k):
        p = L - k + i
        lo = max(0, p + 1 - W)
        scores = [scale * math.fsum(a * b for a, b in zip(Q[i], K[j])) for j in range(lo, p + 1)]
        top = max(scores)
        w = [math.exp(s - top) for s in scores]
        z = math.fsum(w)
        out.append([math.fsum(w[j] * V[lo + j][d] for j in range(len(w))) / z for d in range(len(V[0]))])
    return out


@pytest.mark.parametrize("k,W,R", [(1, 33, 3), (4, 30, 3), (3, 47, 4), (2, 1, 2)])
def test_window_chunks_brute_force(k, W, R):
    """Each query of a chunk over a wrapped ring sees only the window ending at
    itself: the textbook with per-query bounds on the contiguous K/V."""
    rng = np.random.default_rng(7 * k + W)
    B, Hkv, G, D, P = 2, 2, 2, 32, 16
    Hq = Hkv * G
    lens = np.array([k + 3, R * P * 3 + 9], np.int32)
    ring, kp, vp, K, V = _ring_case(rng, B, Hkv, D, P, R, lens)
    q = rng.standard_normal((B, k, Hq, D)).astype(np.float16)
    got = oracle.decode_attention_window_multi(q, kp, vp, ring, lens, W, 0.2, P)
    s32 = float(np.float32(0.2))
    for b in range(B):
        for h in range(Hq):
            kvh = h // G
            ref = _window_causal_textbook(q[b, :, h].astype(float).tolist(), K[b][kvh].astype(float).tolist(),
                                          V[b][kvh].astype(float).tolist(), s32, W)
            np.testing.assert_allclose(got[b, :, h], ref, rtol=0, atol=1e-12)
    one = oracle.decode_attention_window_multi(q[:, -1:], kp, vp, ring, lens, W, 0.2, P)
    np.testing.assert_array_equal(one[:, 0], oracle.decode_attention_window(q[:, -1], kp, vp, ring, lens, W, 0.2, P))
    short = oracle.decode_attention_window_multi(q, kp, vp, ring, np.array([k - 1, 40], np.int32), W, 0.2, P)
    if k > 1:
        assert np.all(np.isnan(short[0])) and np.all(np.isfinite(short[1]))
    idle = oracle.decode_attention_window_multi(q, kp, vp, ring, np.array([0, 40], np.int32), W, 0.2, P)
    assert np.all(idle[0] == 0) and np.array_equal(idle[1], short[1])
