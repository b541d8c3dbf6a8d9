"""Seeded synthetic decode workloads shared by the tests and the bench.

This module only draws inputs. It holds none of the attention or append
arithmetic, and imports neither the oracle nor the HIP package.

Recipe (same in tests and bench):
* ``seed`` = workload number unless given; ``numpy.random.default_rng(seed)``
  (PCG64) draws, in order, the context lengths and then the pool page
  permutation;
* values: float32 N(0, 1) rounded to fp16, filling every pool slot; array ``a``
  (q=1, K pool=2, V pool=3, new K=4, new V=5) is drawn in chunks of 2^20 values,
  chunk ``c`` from PCG64 seeded with ``SeedSequence([seed, a, c])``;
* pages of each sequence are consecutive entries of the permutation, so
  logical neighbours sit at random physical pages.

Workloads (shapes of the attention layers of the models the pages discuss --
Qwen/Llama-2-7B MHA and Llama-3-8B GQA; request lengths of a few hundred up to a
few thousand tokens as on dpshk §2.1):

1. tiny: B=1, Hq=Hkv=4, D=64, 256 tokens, P=16, the 16 pages at the first 16
   entries of a permutation of a 64-page pool, scale 1/8, no append.
2. llama2-7b-mha: B=8, Hq=Hkv=32, D=128, cached context ~ U{200..4096}, P=16,
   pool sized to the demand, append one token then attend over context+1;
   1024-token partitions (the split path: 8 sequences alone fill too few
   workgroups).
3. llama3-8b-gqa-prefix: B=64, Hq=32, Hkv=8, D=128, P=16; every sequence starts
   with the same 128 pages (a 2048-token system prefix); private context
   ~ round(LogNormal(ln 1024, ln 2)) clipped to [128, 8192]; append one token;
   1024-token partitions.
4. long-context: B=4, Hq=32, Hkv=8, D=128, 32767 cached tokens + 1 appended
   = 32768, P=16, split into 512-token partitions.
5. page-sweep: B=32, Hq=32, Hkv=8, D=128, cached context ~ U{200..4000},
   P in {16, 32, 64, 128}, 64 consecutive append+decode steps; pages for all 64
   steps reserved up front; 512-token partitions.
6. sliding-window-4096: B=32, Hq=32, Hkv=8, D=128, P=16, a 4096-token window
   over a ring of 257 pages per sequence (the most pages a 4096-token window
   touches), cached context ~ U{4096..32768} (the ring has wrapped up to eight
   times), append one token; ``block_table`` is the ring table [B][257] drawn
   as consecutive entries of the permutation of the B * 257 pages; unsplit
   (once every window is full, each (sequence, KV head) carries the same 4096
   tokens: 256 equal workgroups, one per compute unit).
"""

import math
import os
from dataclasses import dataclass, field

import numpy as np

PREFIX_PAGES_W3 = 128


@dataclass
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    N: int
    scale: float
    q: np.ndarray            # fp16 [B][Hq][D]
    k_pool: np.ndarray       # fp16 storage [N][Hkv][P/16][16*D] (tile layout of the oracle)
    v_pool: np.ndarray       # fp16 storage [N][Hkv][P/16][16*D]
    block_table: np.ndarray  # int32 [B][max_pages], -1 where unused
    context: np.ndarray      # int32 [B] tokens cached before the first step
    k_new: np.ndarray        # fp16 [steps][B][Hkv][D] (steps may be 0)
    v_new: np.ndarray        # fp16 [steps][B][Hkv][D]
    partition_tokens: int = 0
    shared_prefix_pages: int = 0
    perm: np.ndarray = field(default=None, repr=False)
    window: int = 0          # > 0: attend the last `window` tokens; block_table is a ring of pages

    @property
    def steps(self):
        return int(self.k_new.shape[0])

    @property
    def max_pages(self):
        return int(self.block_table.shape[1])

    def pos(self, step):
        """Position the new token of ``step`` is written at, per sequence."""
        return (self.context + step).astype(np.int32)

    def lens(self, step):
        """Context attended by ``step`` (the appended token included)."""
        if self.steps == 0:
            return self.context.astype(np.int32)
        return (self.context + step + 1).astype(np.int32)


_CHUNK = 1 << 20
_POOL = None


def _normal_fp16(seed, array_id, shape):
    """fp16 N(0,1) array; chunk ``c`` of it comes from the PCG64 stream seeded by
    ``SeedSequence([seed, array_id, c])`` (float32 normals rounded to fp16), so the
    values do not depend on how many threads draw them."""
    global _POOL
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16)

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, array_id, c])))
        out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)

    n_chunks = -(-n // _CHUNK)
    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        if _POOL is None:
            from concurrent.futures import ThreadPoolExecutor
            _POOL = ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0)))))
        list(_POOL.map(fill, range(n_chunks)))
    return out.reshape(shape)


def _ceil_div(a, b):
    return -(-a // b)


def _build(name, rng, seed, B, Hq, Hkv, D, P, context, tokens_needed, steps, scale,
           prefix_pages=0, extra_pool_pages=0, partition_tokens=0):
    """Lay pages out through a random permutation and draw the values."""
    private_pages = [_ceil_div(int(t), P) - prefix_pages for t in tokens_needed]
    n_pages = prefix_pages + sum(private_pages) + extra_pool_pages
    perm = rng.permutation(n_pages).astype(np.int32)
    width = max(prefix_pages + pp for pp in private_pages)
    bt = np.full((B, width), -1, dtype=np.int32)
    cursor = prefix_pages
    for b in range(B):
        bt[b, :prefix_pages] = perm[:prefix_pages]
        bt[b, prefix_pages:prefix_pages + private_pages[b]] = perm[cursor:cursor + private_pages[b]]
        cursor += private_pages[b]
    q = _normal_fp16(seed, 1, (B, Hq, D))
    k_pool = _normal_fp16(seed, 2, (n_pages, Hkv, P // 16, 16 * D))
    v_pool = _normal_fp16(seed, 3, (n_pages, Hkv, P // 16, 16 * D))
    k_new = _normal_fp16(seed, 4, (steps, B, Hkv, D))
    v_new = _normal_fp16(seed, 5, (steps, B, Hkv, D))
    return DecodeWorkload(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, P=P, N=n_pages, scale=scale,
                          q=q, k_pool=k_pool, v_pool=v_pool, block_table=bt,
                          context=np.asarray(context, dtype=np.int32), k_new=k_new, v_new=v_new,
                          partition_tokens=partition_tokens, shared_prefix_pages=prefix_pages,
                          perm=perm)


def workload(number, page_size=None, seed=None, batch=None):
    """Build workload ``number`` (1..6). ``page_size`` applies to workload 5
    (default 16); ``batch`` shrinks B for quick tests (same recipe)."""
    seed = number if seed is None else seed
    rng = np.random.default_rng(seed)
    if number == 1:
        B, Hq, Hkv, D, P = 1, 4, 4, 64, 16
        B = batch or B
        context = np.full(B, 256, dtype=np.int64)
        # tiny case: 16 pages per sequence out of a 64-page pool per sequence
        n_pages = 64 * B
        perm = rng.permutation(n_pages).astype(np.int32)
        bt = np.stack([perm[16 * b:16 * b + 16] for b in range(B)]).astype(np.int32)
        q = _normal_fp16(seed, 1, (B, Hq, D))
        k_pool = _normal_fp16(seed, 2, (n_pages, Hkv, P // 16, 16 * D))
        v_pool = _normal_fp16(seed, 3, (n_pages, Hkv, P // 16, 16 * D))
        empty = np.zeros((0, B, Hkv, D), dtype=np.float16)
        return DecodeWorkload("tiny", B, Hq, Hkv, D, P, n_pages, 1.0 / math.sqrt(D), q, k_pool, v_pool,
                              bt, context.astype(np.int32), empty, empty.copy(), perm=perm)
    if number == 2:
        B = batch or 8
        ctx = rng.integers(200, 4096, size=B, endpoint=True)
        return _build("llama2-7b-mha", rng, seed, B, 32, 32, 128, 16, ctx, ctx + 1, 1, 1.0 / math.sqrt(128),
                      partition_tokens=1024)
    if number == 3:
        B = batch or 64
        private = np.clip(np.rint(rng.lognormal(math.log(1024.0), math.log(2.0), size=B)), 128, 8192).astype(np.int64)
        ctx = PREFIX_PAGES_W3 * 16 + private
        return _build("llama3-8b-gqa-prefix", rng, seed, B, 32, 8, 128, 16, ctx, ctx + 1, 1, 1.0 / math.sqrt(128),
                      prefix_pages=PREFIX_PAGES_W3, partition_tokens=1024)
    if number == 4:
        B = batch or 4
        ctx = np.full(B, 32767, dtype=np.int64)
        return _build("long-context", rng, seed, B, 32, 8, 128, 16, ctx, ctx + 1, 1, 1.0 / math.sqrt(128),
                      partition_tokens=512)
    if number == 5:
        B = batch or 32
        P = page_size or 16
        steps = 64
        ctx = rng.integers(200, 4000, size=B, endpoint=True)
        return _build("page-sweep-p%d" % P, rng, seed, B, 32, 8, 128, P, ctx, ctx + steps, steps,
                      1.0 / math.sqrt(128), partition_tokens=512)
    if number == 6:
        B = batch or 32
        P, W = 16, 4096
        R = (W - 1) // P + 2
        ctx = rng.integers(W, 8 * W, size=B, endpoint=True)
        n_pages = B * R
        perm = rng.permutation(n_pages).astype(np.int32)
        ring = perm.reshape(B, R).copy()
        q = _normal_fp16(seed, 1, (B, 32, 128))
        k_pool = _normal_fp16(seed, 2, (n_pages, 8, P // 16, 16 * 128))
        v_pool = _normal_fp16(seed, 3, (n_pages, 8, P // 16, 16 * 128))
        k_new = _normal_fp16(seed, 4, (1, B, 8, 128))
        v_new = _normal_fp16(seed, 5, (1, B, 8, 128))
        return DecodeWorkload("sliding-window-4096", B, 32, 8, 128, P, n_pages, 1.0 / math.sqrt(128), q, k_pool,
                              v_pool, ring, ctx.astype(np.int32), k_new, v_new, partition_tokens=0, perm=perm,
                              window=W)
    raise ValueError("workload number must be 1..6")
