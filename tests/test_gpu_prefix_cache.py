"""GPU side of the prefix-cache lifecycle: page copies are byte-exact, and a
copy-on-write step (two sequences sharing a cached prompt whose last page is
partly filled both append into it) decodes exactly as the oracle does on the
same logical caches."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import PageAllocatorModel

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def pkv():
    import paged_kv_cache_279_amd as m
    m.lib()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("shape", [(40, 8, 16, 128), (9, 2, 64, 64), (200, 8, 16, 128)])
def test_copy_pages_byte_exact(shape):
    rng = np.random.default_rng(shape[0])
    pool = rng.standard_normal(shape).astype(np.float16)
    N = shape[0]
    perm = rng.permutation(N)
    n = min(N // 2, 100)                       # more than one launch of 64 pairs for the big pool
    src, dst = perm[:n], perm[n:2 * n]
    d = dev(pool)
    say("copy pages", shape, n)
    pkv().copy_pages(d, src, dst)
    torch.cuda.synchronize()
    expect = pool.copy()
    expect[dst] = pool[src]
    assert np.array_equal(host(d).view(np.uint16), expect.view(np.uint16))


def test_copy_on_write_decode_matches_oracle():
    m = pkv()
    rng = np.random.default_rng(8)
    N, Hkv, G, P, D = 24, 2, 4, 16, 128
    Hq = Hkv * G
    prompt = 40                                     # 2.5 pages: the third page is partly filled
    a = m.PageAllocator(N, P)
    model = PageAllocatorModel(N, P)
    kp = rng.standard_normal(oracle.pool_shape(N, Hkv, P, D)).astype(np.float16)
    vp = rng.standard_normal(oracle.pool_shape(N, Hkv, P, D)).astype(np.float16)
    # sequence 0 holds the prompt; the cache keeps it; sequences 1 and 2 start from the cache
    for alloc in (a, model):
        alloc.reserve(0, prompt)
        alloc.cache_insert(11, 0, prompt)
    pages, n_tok = a.cache_lookup(11)
    assert (pages, n_tok) == (model.cache_lookup(11)[0], prompt)
    for s in (1, 2):
        a.share_prefix(s, pages)
        model.share_prefix(s, pages)
    a.free(0)
    model.free(0)
    # both write token 40, inside the shared third page
    B = 2
    seqs = np.array([1, 2], np.int32)
    pos = np.array([prompt, prompt], np.int32)
    bt = np.full((B, 4), -1, np.int32)
    copies = a.prepare_append(seqs, pos, bt)
    assert copies == model.prepare_append(seqs, pos)
    assert len(copies) == 2                          # the cache still holds the page: both sharers copy
    kd, vd = dev(kp), dev(vp)
    m.copy_pages(kd, [c[0] for c in copies], [c[1] for c in copies])
    m.copy_pages(vd, [c[0] for c in copies], [c[1] for c in copies])
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    lens = pos + 1
    out = m.append_paged_decode_attention(dev(q), dev(kn), dev(vn), kd, vd, dev(bt), dev(lens), int(lens.max()),
                                          1 / math.sqrt(D), 0)
    torch.cuda.synchronize()
    # oracle: the same steps on host copies
    ko, vo = kp.copy(), vp.copy()
    for src, dst in copies:
        ko[dst] = ko[src]
        vo[dst] = vo[src]
    ko, vo = oracle.kv_append(ko, vo, kn, vn, bt, pos, P)
    assert np.array_equal(host(kd).view(np.uint16), ko.view(np.uint16))
    assert np.array_equal(host(vd).view(np.uint16), vo.view(np.uint16))
    ref = oracle.decode_attention(q, ko, vo, bt, lens, 1 / math.sqrt(D), P)
    err = np.abs(host(out).astype(np.float64) - ref).max()
    say("copy-on-write decode: max_abs_err=%.3e" % err)
    assert err <= 4e-3
    # the cached prompt is untouched: its third page still holds the original tokens
    cached, _ = a.cache_lookup(11)
    assert np.array_equal(host(kd)[cached[2]].view(np.uint16), kp[cached[2]].view(np.uint16))
