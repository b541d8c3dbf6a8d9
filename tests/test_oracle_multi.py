"""Pins for the multi-query (chunk / draft verification) oracle.

* brute force: a textbook causal attention that scores every query against
  every key of the contiguous K/V and masks the future (an upper-triangular
  mask on the k x L score matrix), against the oracle reading the same K/V
  through permuted pages;
* k = 1 is single-token decode;
* the last query of a chunk is the decode step of the whole sequence, the
  first query ignores the k - 1 newer keys (changing them moves only the later
  queries).
"""

import math

import numpy as np
import pytest

import oracle
from test_oracle_pins import make_paged_case


def causal_textbook(Q, K, V, scale):
    """Q [k][D], K/V [L][D] (contiguous): scores S = scale Q K^T, query i may
    see keys j <= L - k + i, softmax over what it may see, weighted sum of V."""
    k, L = len(Q), len(K)
    out = []
    for i in range(k):
        scores = []
        for j in range(L):
            s = scale * math.fsum(a * b for a, b in zip(Q[i], K[j]))
            scores.append(s if j <= L - k + i else -math.inf)
        top = max(scores)
        w = [math.exp(s - top) if s != -math.inf else 0.0 for s in scores]
        z = math.fsum(w)
        out.append([math.fsum(w[j] * V[j][d] for j in range(L)) / z for d in range(len(V[0]))])
    return out


@pytest.mark.parametrize("k,G,P", [(1, 2, 16), (2, 4, 16), (4, 4, 32), (3, 1, 16), (16, 1, 16)])
def test_multi_query_brute_force(k, G, P):
    rng = np.random.default_rng(17 * k + G)
    B, Hkv, D = 2, 2, 32
    Hq = Hkv * G
    lens = np.array([k + 5, k + 37], np.int32)
    q_unused, kp, vp, bt, K, V = make_paged_case(rng, B, Hq, Hkv, D, P, lens)
    q = rng.standard_normal((B, k, Hq, D)).astype(np.float16)
    got = oracle.decode_attention_multi(q, kp, vp, bt, lens, 0.4, P)
    s32 = float(np.float32(0.4))
    for b in range(B):
        for h in range(Hq):
            kvh = h // G
            ref = causal_textbook(q[b, :, h].astype(float).tolist(), K[b][kvh].astype(float).tolist(),
                                  V[b][kvh].astype(float).tolist(), s32)
            np.testing.assert_allclose(got[b, :, h], ref, rtol=0, atol=1e-12)


def test_single_query_is_decode():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, P = 3, 4, 2, 32, 16
    lens = np.array([1, 20, 47], np.int32)
    q, kp, vp, bt, K, V = make_paged_case(rng, B, Hq, Hkv, D, P, lens)
    got = oracle.decode_attention_multi(q[:, None], kp, vp, bt, lens, 0.25, P)
    ref = oracle.decode_attention(q, kp, vp, bt, lens, 0.25, P)
    assert np.array_equal(got[:, 0], ref)


def test_causality_within_the_chunk():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, D, P, k = 2, 4, 2, 32, 16, 4
    lens = np.array([30, 51], np.int32)
    q, kp, vp, bt, K, V = make_paged_case(rng, B, Hq, Hkv, D, P, lens, poison=False)
    qm = rng.standard_normal((B, k, Hq, D)).astype(np.float16)
    base = oracle.decode_attention_multi(qm, kp, vp, bt, lens, 0.3, P)
    # the last query is the full decode step
    np.testing.assert_allclose(base[:, -1], oracle.decode_attention(qm[:, -1], kp, vp, bt, lens, 0.3, P), atol=0)
    # overwrite the newest key of every sequence: only the last query may change
    kp2 = kp.copy()
    for b in range(B):
        t = int(lens[b]) - 1
        for h in range(Hkv):
            oracle.write_token(kp2, bt[b, t // P], h, t % P, rng.standard_normal(D).astype(np.float16), "k")
    moved = oracle.decode_attention_multi(qm, kp2, vp, bt, lens, 0.3, P)
    assert np.array_equal(moved[:, :-1], base[:, :-1])
    assert not np.allclose(moved[:, -1], base[:, -1])
    # a sequence shorter than the chunk is an invalid row: all of it NaN, the others untouched
    short = lens.copy()
    short[0] = 2
    nanrows = oracle.decode_attention_multi(qm, kp, vp, bt, short, 0.3, P)
    assert np.all(np.isnan(nanrows[0])) and np.array_equal(nanrows[1], base[1])
    # length 0 is an idle batch slot: zero rows, the others untouched
    short[0] = 0
    idle = oracle.decode_attention_multi(qm, kp, vp, bt, short, 0.3, P)
    assert np.all(idle[0] == 0) and np.array_equal(idle[1], base[1])
