"""fp64 reference for the paged KV store, in-place append and decode attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

Data format (the pages give a page as "tokens x heads x dims" in fp16 without
fixing the axis order -- hotelren §3.2, pgsm §3.2; the order below is this
library's reading):

* ``k_pool``, ``v_pool``: fp16 arrays of storage shape ``[N][Hkv][P/16][16*D]``
  (``pool_shape``): N pages x Hkv KV heads x P/16 sub-blocks of 16 tokens; the
  ``P*D`` halves of one (page, kv head) tile are contiguous. Inside a tile,
  token ``t`` and dim ``d`` sit at the offset given by ``k_tile_offset`` /
  ``v_tile_offset`` (K keeps 8-dim chunks with the token index minor, V keeps
  4-token groups with the token index minor), so a sub-block is storage, not a
  (token, dim) array.
* ``block_table``: int32 ``[B][max_pages]``; entry ``j`` of row ``b`` is the
  physical page holding logical tokens ``j*P .. j*P+P-1`` of sequence ``b``
  (pgsm §3.2 and §4.1: a page table maps each sequence's pages).
* ``lens``: int32 ``[B]``, tokens of context per sequence *including* the token
  appended this step.
* query head ``h`` reads KV head ``h // (Hq // Hkv)`` (grouped-query sharing; the
  pages only say a layer has H KV heads, dpshk §4.1).

Arithmetic is float64 throughout; fp16 inputs widen exactly.
"""

import math

import numpy as np


# ---------------------------------------------------------------------------
# sizes
# ---------------------------------------------------------------------------

def kv_cache_bytes(layers, kv_heads, head_dim, seq_len, dtype_bytes=2, batch=1):
    """Bytes of K plus V for ``batch`` sequences of ``seq_len`` tokens.

    dpshk §4.1 gives the size as 2 (K and V) x layers x heads x head_dim x
    tokens x 2 bytes (fp16); pgsm §4.1 states the same product with a batch
    factor.
    """
    return 2 * batch * layers * kv_heads * head_dim * seq_len * dtype_bytes


def pages_for_tokens(n_tokens, page_size):
    """Pages needed to hold ``n_tokens`` tokens: the ceiling of n / P.

    pgsm §4.1 tabulates pages per request against page size for ~2048-token
    requests (128, 64, 32, 16 pages at P = 16, 32, 64, 128).
    """
    if n_tokens < 0 or page_size <= 0:
        raise ValueError("n_tokens must be >= 0 and page_size > 0")
    return -(-n_tokens // page_size)


def pool_bytes(num_pages, kv_heads, page_size, head_dim, dtype_bytes=2):
    """Bytes of one layer's K pool plus V pool ``[N][Hkv][P][D]`` each."""
    return 2 * num_pages * kv_heads * page_size * head_dim * dtype_bytes


# ---------------------------------------------------------------------------
# paging
# ---------------------------------------------------------------------------

def token_slot(block_table_row, t, page_size):
    """Physical (page, token-in-page) of logical token ``t``.

    The page table lookup of pgsm §3.2: logical page ``t // P`` is looked up in
    the sequence's table; the token is number ``t % P`` inside that page.
    """
    page = int(block_table_row[t // page_size])
    return page, t % page_size


def _check_tile(page_size, head_dim):
    if page_size % 16 or head_dim % 32 or page_size <= 0 or head_dim <= 0:
        raise ValueError("tile layout needs page_size % 16 == 0 and head_dim % 32 == 0")


def k_tile_offset(t, d, page_size, head_dim):
    """Offset (in halves) of token ``t`` (within its page), dim ``d`` in a K tile.

    16-token sub-block ``t // 16``; inside it, dim chunk ``d // 8`` is a run of
    16 tokens x 8 dims: offset ``((d // 8) * 16 + t % 16) * 8 + d % 8``.
    """
    _check_tile(page_size, head_dim)
    t = np.asarray(t)
    d = np.asarray(d)
    return (t // 16) * 16 * head_dim + ((d // 8) * 16 + t % 16) * 8 + d % 8


def v_tile_offset(t, d, page_size, head_dim):
    """Offset (in halves) of token ``t`` (within its page), dim ``d`` in a V tile.

    16-token sub-block ``t // 16``; inside it the 4-token group ``(t % 16) // 4``
    of 32-dim slice ``d // 32`` holds, for each of 16 dims ``d % 16``, the two
    16-dim halves of the slice (``(d // 16) % 2``) with 4 tokens each.
    """
    _check_tile(page_size, head_dim)
    t = np.asarray(t)
    d = np.asarray(d)
    u = t % 16
    return ((t // 16) * 16 * head_dim
            + (((d // 32) * 4 + u // 4) * 16 + d % 16) * 8 + ((d // 16) % 2) * 4 + u % 4)


def _tile_offset(kind, t, d, page_size, head_dim):
    if kind == "k":
        return k_tile_offset(t, d, page_size, head_dim)
    if kind == "v":
        return v_tile_offset(t, d, page_size, head_dim)
    raise ValueError("kind must be 'k' or 'v'")


def pool_shape(num_pages, kv_heads, page_size, head_dim):
    """Storage shape of a K or V pool: ``[N][Hkv][P/16][16*D]``."""
    _check_tile(page_size, head_dim)
    return (num_pages, kv_heads, page_size // 16, 16 * head_dim)


def pool_dims(pool):
    """``(N, Hkv, P, D)`` of a pool of storage shape ``[N][Hkv][P/16][16*D]``."""
    n, hkv, nsub, width = pool.shape
    if width % 16:
        raise ValueError("a pool's last axis holds 16 tokens x D halves")
    return n, hkv, 16 * nsub, width // 16


def _tiles(pool):
    n, hkv, p, d = pool_dims(pool)
    return pool.reshape(n, hkv, p * d)


def read_token(pool, page, kv_head, t, kind):
    """The ``D`` halves of token ``t`` (within ``page``) of one KV head."""
    n, hkv, p, dim = pool_dims(pool)
    return _tiles(pool)[page, kv_head, _tile_offset(kind, t, np.arange(dim), p, dim)]


def write_token(pool, page, kv_head, t, vec, kind):
    """Store the ``D`` halves ``vec`` as token ``t`` of ``page`` (in place)."""
    n, hkv, p, dim = pool_dims(pool)
    _tiles(pool)[page, kv_head, _tile_offset(kind, t, np.arange(dim), p, dim)] = vec


def gather_sequence(pool, block_table_row, length, kv_head, page_size, kind):
    """Contiguous float64 ``[length][D]`` copy of one sequence's K or V.

    Token ``t`` is read from page ``block_table_row[t // P]`` as token
    ``t % P`` of that page (``token_slot``), through the tile layout of
    ``kind``, so the result is exactly the contiguous cache a non-paged
    implementation would hold.
    """
    n, hkv, p, dim = pool_dims(pool)
    if p != page_size:
        raise ValueError("pool page size differs from page_size")
    t = np.arange(length)
    pages = np.asarray(block_table_row, dtype=np.int64)[t // page_size]
    if length and (pages.min() < 0 or pages.max() >= n):
        raise IndexError("block table entry out of range")
    off = _tile_offset(kind, (t % page_size)[:, None], np.arange(dim)[None, :], page_size, dim)
    return _tiles(pool)[pages[:, None], kv_head, off].astype(np.float64)


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------

def _scale64(scale):
    # the scale reaches the library as a 32-bit float; widen that exact value
    return float(np.float32(scale))


def _check_heads(hq, hkv):
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    return hq // hkv


def decode_attention(q, k_pool, v_pool, block_table, lens, scale, page_size):
    """One decode step of attention for every sequence and query head.

    For sequence ``b`` and query head ``h`` (KV head ``h // g``):
    gather the ``lens[b]`` past keys/values through the page table, score
    ``s_t = scale * <q, k_t>``, normalise with a softmax, and return the
    softmax-weighted sum of the values (pgsm §4.2: a decode step reads all
    past KV, scores them, normalises and takes the weighted sum).

    ``lens[b] == 0`` yields a zero row (there is nothing to attend to).
    Returns float64 ``[B][Hq][D]``.
    """
    b_count, hq, d = q.shape
    hkv = k_pool.shape[1]
    g = _check_heads(hq, hkv)
    s64 = _scale64(scale)
    out = np.zeros((b_count, hq, d), dtype=np.float64)
    for b in range(b_count):
        n = int(lens[b])
        if n == 0:
            continue
        for kvh in range(hkv):
            keys = gather_sequence(k_pool, block_table[b], n, kvh, page_size, "k")
            vals = gather_sequence(v_pool, block_table[b], n, kvh, page_size, "v")
            for i in range(g):
                h = kvh * g + i
                qh = q[b, h].astype(np.float64)
                s = s64 * (keys @ qh)
                p = np.exp(s - s.max())
                out[b, h] = (p @ vals) / p.sum()
    return out


def decode_attention_window(q, k_pool, v_pool, ring_table, lens, window, scale, page_size):
    """Decode attention over the last ``window`` tokens, pages kept in a ring.

    The static, fixed-capacity variant of the KV cache (hotelren §3.2: a ring
    buffer of preallocated storage that overwrites its oldest entries) expressed
    through the page table: sequence ``b`` owns ``R = ring_table.shape[1]``
    pages, and logical page ``j`` lives in page ``ring_table[b][j % R]``, so a
    new page overwrites the one ``R`` pages older. Query ``b`` attends tokens
    ``max(0, lens[b] - window) .. lens[b] - 1`` (the window must fit in the
    ring: ``window <= (R - 1) * P + 1``); token ``t`` is slot ``t % P`` of page
    ``ring_table[b][(t // P) % R]``. Otherwise exactly ``decode_attention``.
    Returns float64 ``[B][Hq][D]``; ``lens[b] == 0`` gives zeros.
    """
    b_count, hq, d = q.shape
    n, hkv, p, dim = pool_dims(k_pool)
    ring = np.asarray(ring_table, dtype=np.int64)
    r = ring.shape[1]
    if window <= 0 or window > (r - 1) * page_size + 1:
        raise ValueError("the window must fit in the ring")
    g = _check_heads(hq, hkv)
    s64 = _scale64(scale)
    out = np.zeros((b_count, hq, d), dtype=np.float64)
    for b in range(b_count):
        length = int(lens[b])
        if length == 0:
            continue
        t = np.arange(max(0, length - window), length)
        pages = ring[b][(t // page_size) % r]
        slots = (t % page_size)[:, None]
        for kvh in range(hkv):
            keys = _tiles(k_pool)[pages[:, None], kvh, k_tile_offset(slots, np.arange(dim)[None, :], p, dim)]
            vals = _tiles(v_pool)[pages[:, None], kvh, v_tile_offset(slots, np.arange(dim)[None, :], p, dim)]
            keys = keys.astype(np.float64)
            vals = vals.astype(np.float64)
            for i in range(g):
                h = kvh * g + i
                sc = s64 * (keys @ q[b, h].astype(np.float64))
                w = np.exp(sc - sc.max())
                out[b, h] = (w @ vals) / w.sum()
    return out


def decode_attention_multi(q, k_pool, v_pool, block_table, lens, scale, page_size):
    """Attention for the last ``k`` tokens of every sequence at once.

    ``q`` is ``[B][k][Hq][D]``: the queries of a sequence's last ``k`` positions
    ``lens[b] - k .. lens[b] - 1``, whose keys and values are already in the
    cache. Each query attends causally: query ``i`` sees tokens
    ``0 .. lens[b] - k + i``. This is the attention of verifying ``k`` drafted
    tokens in one pass or of one chunk of a chunked prefill (pgsm §3.2 names
    both: speculative decoding checks several candidate tokens in parallel,
    chunked prefill processes a prompt in pieces over the paged cache); each
    query is exactly a single-token decode step over its own prefix, so it is
    computed as one (``decode_attention`` with length ``lens[b] - k + i + 1``).
    Returns float64 ``[B][k][Hq][D]``; a row whose query would start before
    token 0 (``0 < lens[b] < k``) is all NaN; ``lens[b] == 0`` (an idle batch
    slot) gives zeros.
    """
    b_count, k, hq, d = q.shape
    out = np.zeros((b_count, k, hq, d), dtype=np.float64)
    lens64 = np.asarray(lens, dtype=np.int64)
    # the chunk would reach before token 0: the whole row is invalid; length 0 is an idle slot (zeros)
    short = (lens64 < k) & (lens64 != 0)
    for i in range(k):
        li = np.where(lens64 < k, 0, lens64 - k + i + 1)
        out[:, i] = decode_attention(q[:, i], k_pool, v_pool, block_table, li, scale, page_size)
    out[short] = np.nan
    return out


def decode_attention_window_multi(q, k_pool, v_pool, ring_table, lens, window, scale, page_size):
    """Chunks of queries over a sliding window in a ring of pages: query ``i``
    of sequence ``b`` sits at position ``p = lens[b] - k + i`` (the chunk
    reading of ``decode_attention_multi``) and attends the last ``window``
    tokens up to itself, ``max(0, p + 1 - window) .. p`` (the window reading of
    ``decode_attention_window``), each query being the window decode step of
    its own prefix. All of the chunk's tokens must still be in the ring:
    ``window + k - 1 <= (R - 1) * P + 1``. Returns float64 ``[B][k][Hq][D]``; a
    row with ``0 < lens[b] < k`` is all NaN; ``lens[b] == 0`` gives zeros."""
    b_count, k, hq, d = q.shape
    r = np.asarray(ring_table).shape[1]
    if window + k - 1 > (r - 1) * page_size + 1:
        raise ValueError("the chunk's windows must fit in the ring")
    out = np.zeros((b_count, k, hq, d), dtype=np.float64)
    lens64 = np.asarray(lens, dtype=np.int64)
    short = (lens64 < k) & (lens64 != 0)        # length 0: an idle slot (zeros)
    for i in range(k):
        li = np.where(lens64 < k, 0, lens64 - k + i + 1)
        out[:, i] = decode_attention_window(q[:, i], k_pool, v_pool, ring_table, li, window, scale, page_size)
    out[short] = np.nan
    return out


def kv_append(k_pool, v_pool, k_new, v_new, block_table, pos, page_size):
    """Return copies of the pools with each sequence's new token written.

    Decode only appends the new token's K and V (one ``D``-vector per KV head
    each) at position ``pos[b]`` and never rewrites older entries (pgsm §3.2 and
    §4.3; hotelren §3.1 appends into preallocated storage instead of
    reallocating). The write lands at the slot the page table gives for
    ``pos[b]``.
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    b_count, hkv, _ = k_new.shape
    for b in range(b_count):
        page, off = token_slot(block_table[b], int(pos[b]), page_size)
        for kvh in range(hkv):
            write_token(k_out, page, kvh, off, k_new[b, kvh, :], "k")
            write_token(v_out, page, kvh, off, v_new[b, kvh, :], "v")
    return k_out, v_out


# ---------------------------------------------------------------------------
# split context
# ---------------------------------------------------------------------------

def decode_partials(q, k_pool, v_pool, block_table, lens, scale, page_size,
                    partition_tokens):
    """Per-partition softmax statistics for split-context decode.

    The context of sequence ``b`` is cut into consecutive partitions of
    ``partition_tokens`` tokens (the last may be shorter). For partition ``j``
    and head ``h`` this returns the partition's score maximum ``m``, the sum
    ``l = sum_t exp(s_t - m)`` and the unnormalised ``o = sum_t exp(s_t - m) v_t``.
    The pages do not describe split context; this is the plain reading of the
    standard log-sum-exp decomposition of a softmax.

    Returns a list over ``b`` of tuples ``(m [Hq][n], l [Hq][n], o [Hq][n][D])``.
    """
    if partition_tokens <= 0:
        raise ValueError("partition_tokens must be positive")
    b_count, hq, d = q.shape
    hkv = k_pool.shape[1]
    g = _check_heads(hq, hkv)
    s64 = _scale64(scale)
    result = []
    for b in range(b_count):
        n = int(lens[b])
        n_parts = pages_for_tokens(n, partition_tokens)
        m = np.full((hq, n_parts), -np.inf)
        l = np.zeros((hq, n_parts))
        o = np.zeros((hq, n_parts, d))
        for kvh in range(hkv):
            keys = gather_sequence(k_pool, block_table[b], n, kvh, page_size, "k")
            vals = gather_sequence(v_pool, block_table[b], n, kvh, page_size, "v")
            for i in range(g):
                h = kvh * g + i
                s = s64 * (keys @ q[b, h].astype(np.float64))
                for j in range(n_parts):
                    lo, hi = j * partition_tokens, min(n, (j + 1) * partition_tokens)
                    sj = s[lo:hi]
                    mj = sj.max()
                    pj = np.exp(sj - mj)
                    m[h, j] = mj
                    l[h, j] = pj.sum()
                    o[h, j] = pj @ vals[lo:hi]
        result.append((m, l, o))
    return result


def lse_merge(m, l, o):
    """Merge per-partition statistics of one head into the softmax output.

    With ``M = max_j m_j`` and weights ``w_j = exp(m_j - M)``:
    ``out = sum_j w_j o_j / sum_j w_j l_j``. Exact rearrangement of the
    softmax over the union of the partitions. Empty input gives zeros.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if m.size == 0:
        return np.zeros(o.shape[-1])
    big = m.max()
    w = np.exp(m - big)
    return (w @ o) / float(w @ l)


def fp16_round(x):
    """Round float64 values to the nearest fp16 (ties to even), back as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def max_abs_error(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def rms_error(a, b):
    diff = np.asarray(a, np.float64) - np.asarray(b, np.float64)
    return math.sqrt(float(np.mean(diff * diff))) if diff.size else 0.0
