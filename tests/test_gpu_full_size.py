"""GPU parity at the full sizes of the bench workloads, in the launch
configuration bench.py times: the first decode step of layer 0 (the
workload as drawn), the same entry point, partition size, fused append and
shared-prefix path. Pools are compared byte for byte with the oracle's after
the append; outputs are compared with the oracle within 4e-3 on sampled
sequences (the shortest, the longest, the first, the last and four seeded
others), and every output row must be finite. Slots no sequence attends hold
NaN (paged workloads)."""

import math
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import workload  # noqa: E402
from _helpers import poison_unused  # noqa: E402

TOL = 4e-3


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


def sample_rows(lens, seed):
    rng = np.random.default_rng(seed)
    B = len(lens)
    picks = {0, B - 1, int(np.argmin(lens)), int(np.argmax(lens))}
    picks.update(int(x) for x in rng.choice(B, size=min(B, 4), replace=False))
    return np.array(sorted(picks))


@pytest.mark.parametrize("number,page_size", [(2, None), (3, None), (4, None), (5, 16), (5, 32), (5, 64), (5, 128),
                                              (6, None)])
def test_full_size_first_step_matches_oracle(number, page_size):
    w = workload(number, page_size=page_size)
    m = pkv()
    step = 0
    lens = w.lens(step)
    pos = w.pos(step)
    part = w.partition_tokens
    prefix = w.shared_prefix_pages * w.P
    kn, vn = w.k_new[step], w.v_new[step]
    say("full size %s B=%d P=%d part=%d prefix=%d window=%d" % (w.name, w.B, w.P, part, prefix, w.window))
    if w.window:
        k0, v0 = w.k_pool, w.v_pool
        kd, vd = dev(k0), dev(v0)
        got = m.paged_decode_attention_window(dev(w.q), kd, vd, dev(w.block_table), dev(lens), w.window, w.scale,
                                              part, k_new=dev(kn), v_new=dev(vn))
        width = -(-int(lens.max()) // w.P)
        logical = np.ascontiguousarray(w.block_table[:, np.arange(width) % w.max_pages])
        rk, rv = oracle.kv_append(k0, v0, kn, vn, logical, pos, w.P)
    else:
        # unattended slots (before the append) hold NaN
        k0, v0 = poison_unused(w, lens - 1)
        kd, vd = dev(k0), dev(v0)
        max_context = int(w.lens(max(0, w.steps - 1)).max())
        if prefix:
            got = m.paged_decode_attention_shared_prefix(dev(w.q), kd, vd, dev(w.block_table), dev(lens),
                                                         max_context, w.scale, part, prefix, k_new=dev(kn),
                                                         v_new=dev(vn))
        else:
            got = m.append_paged_decode_attention(dev(w.q), dev(kn), dev(vn), kd, vd, dev(w.block_table), dev(lens),
                                                  max_context, w.scale, part)
        rk, rv = oracle.kv_append(k0, v0, kn, vn, w.block_table, pos, w.P)
    torch.cuda.synchronize()
    assert np.array_equal(host(kd).view(np.uint16), rk.view(np.uint16)), "K pool after the append"
    assert np.array_equal(host(vd).view(np.uint16), rv.view(np.uint16)), "V pool after the append"
    out = host(got).astype(np.float64)
    assert np.all(np.isfinite(out)), "non-finite output rows"
    rows = sample_rows(lens, 1000 + number)
    if w.window:
        ref = oracle.decode_attention_window(w.q[rows], rk, rv, w.block_table[rows], lens[rows], w.window, w.scale,
                                             w.P)
    else:
        ref = oracle.decode_attention(w.q[rows], rk, rv, w.block_table[rows], lens[rows], w.scale, w.P)
    err = np.abs(out[rows] - ref)
    say("%s rows %s: max_abs_err=%.3e rms=%.3e" % (w.name, rows.tolist(), err.max(),
                                                 math.sqrt(float((err ** 2).mean()))))
    assert err.max() <= TOL
