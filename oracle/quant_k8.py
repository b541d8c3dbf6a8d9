"""fp64 reference for key-only int8 KV pages.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

What the pages say: quantising the KV cache to int8 halves its memory, but
attention loses precision on long sequences; the advice is to quantise only
the keys and keep the values in high precision (dpshk §4.4), and to quantise
block-wise rather than whole tensors (pgsm §4.2). The pages fix neither the
block nor the rounding, so this library reads them as follows:

* the block is one token's ``D`` key values of one KV head: each gets its own
  fp32 scale. Appends write a token once and never touch older tokens
  (pgsm §4.3), so a scale shared by a whole page would have to be fixed before
  the page's later tokens exist (clipping them) or rewritten with them;
* symmetric int8: ``scale = amax / 127`` and ``code = rint(k * (127 / amax))``
  with round-half-to-even, in IEEE fp32 arithmetic (the kernel's precision:
  where a float decides an integer, both sides decide it the same way); the
  reciprocal ``127 / amax`` is rounded to fp32 once per token, so a kernel
  needs one division per token rather than one per element; ``amax == 0``
  gives scale 0 and all-zero codes;
* the dequantised key is ``code * scale``; attention is then computed exactly
  as for fp16 keys (``decode_attention``), in fp64.

Storage (this library's format): the K pool is bytes
``[N][Hkv][P / 16][16 * D + 64]``; one 16-token sub-block holds the 16 x D
codes followed by the 16 fp32 scales (little-endian, token ``u`` at byte
``16 * D + 4 * u``). Code (token ``u``, dim ``d``) sits at byte
``((d // 64) * 64 + ((d // 8) % 4) * 16 + u) * 16 + ((d // 32) % 2) * 8 + d % 8``:
per 64 dims, 64 runs of 16 bytes, run ``quad * 16 + u`` holding dims
``32 j + 8 quad .. + 8`` of token ``u`` for the two 32-dim slices ``j`` of those
64 dims. The V pool is the fp16 V pool of ``paged_decode``.
"""

import numpy as np

from .paged_decode import _check_heads, _scale64, gather_sequence, token_slot


def k8_subblock_bytes(head_dim):
    """Bytes of one 16-token sub-block of an int8 K tile: codes then scales."""
    if head_dim <= 0 or head_dim % 64:
        raise ValueError("int8 keys need head_dim % 64 == 0")
    return 16 * head_dim + 64


def k8_pool_bytes(num_pages, kv_heads, page_size, head_dim):
    """Bytes of an int8 K pool ``[N][Hkv][P / 16][16 D + 64]``."""
    if page_size <= 0 or page_size % 16:
        raise ValueError("page_size must be a positive multiple of 16")
    return num_pages * kv_heads * (page_size // 16) * k8_subblock_bytes(head_dim)


def k8_code_offset(u, d, head_dim):
    """Byte offset of the code of token ``u`` (0..15), dim ``d`` in a sub-block."""
    k8_subblock_bytes(head_dim)
    u = np.asarray(u)
    d = np.asarray(d)
    return ((d // 64) * 64 + ((d // 8) % 4) * 16 + u) * 16 + ((d // 32) % 2) * 8 + d % 8


def k8_scale_offset(u, head_dim):
    """Byte offset of the fp32 scale of token ``u`` in a sub-block."""
    return 16 * head_dim + 4 * np.asarray(u)


def quantize_k(vec):
    """Symmetric int8 codes and the fp32 scale of one token's key vector.

    ``scale = amax / 127`` and ``code = rint(k * inv)`` (half to even) with
    ``inv = 127 / amax``, each operation in IEEE fp32, so that a kernel doing
    the same fp32 operations reaches the same codes; ``amax == 0`` gives scale
    0 and zero codes.
    """
    k = np.asarray(vec).astype(np.float32)
    amax = np.float32(np.abs(k).max()) if k.size else np.float32(0.0)
    if amax == 0:
        return np.zeros(k.shape, np.int8), np.float32(0.0)
    scale = np.float32(amax / np.float32(127.0))
    inv = np.float32(np.float32(127.0) / amax)
    codes = np.rint(k * inv)
    return np.clip(codes, -127, 127).astype(np.int8), scale


def _subblocks(pool8, head_dim):
    n, hkv, nsub, sb = pool8.shape
    if sb != k8_subblock_bytes(head_dim):
        raise ValueError("sub-block size does not match head_dim")
    return pool8


def k8_write_token(pool8, page, kv_head, t, codes, scale, head_dim):
    """Store token ``t`` (within ``page``): its codes and its scale (in place)."""
    sub = _subblocks(pool8, head_dim)[page, kv_head, t // 16]
    u = t % 16
    sub[k8_code_offset(u, np.arange(head_dim), head_dim)] = np.asarray(codes, np.int8).view(np.uint8)
    so = int(k8_scale_offset(u, head_dim))
    sub[so:so + 4] = np.frombuffer(np.float32(scale).tobytes(), np.uint8)


def k8_read_token(pool8, page, kv_head, t, head_dim):
    """Codes (int8 ``[D]``) and scale (fp32) of token ``t`` within ``page``."""
    sub = _subblocks(pool8, head_dim)[page, kv_head, t // 16]
    u = t % 16
    codes = sub[k8_code_offset(u, np.arange(head_dim), head_dim)].view(np.int8).copy()
    so = int(k8_scale_offset(u, head_dim))
    scale = np.frombuffer(sub[so:so + 4].tobytes(), np.float32)[0]
    return codes, scale


def quantize_k_pool(k_pool):
    """int8 K pool of an fp16 K pool (every slot quantised, tile layout read
    through ``read_token``): ``[N][Hkv][P / 16][16 D + 64]`` bytes."""
    from .paged_decode import pool_dims, read_token
    n, hkv, p, dim = pool_dims(k_pool)
    pool8 = np.zeros((n, hkv, p // 16, k8_subblock_bytes(dim)), np.uint8)
    for page in range(n):
        for h in range(hkv):
            for t in range(p):
                codes, scale = quantize_k(read_token(k_pool, page, h, t, "k"))
                k8_write_token(pool8, page, h, t, codes, scale, dim)
    return pool8


def k8_gather_sequence(pool8, block_table_row, length, kv_head, page_size, head_dim):
    """Dequantised float64 ``[length][D]`` keys of one sequence: token ``t`` is
    read from page ``block_table_row[t // P]`` as token ``t % P`` and becomes
    ``code * scale``."""
    n, hkv, nsub, sb = _subblocks(pool8, head_dim).shape
    if nsub * 16 != page_size:
        raise ValueError("pool page size differs from page_size")
    t = np.arange(length)
    pages = np.asarray(block_table_row, dtype=np.int64)[t // page_size]
    if length and (pages.min() < 0 or pages.max() >= n):
        raise IndexError("block table entry out of range")
    within = t % page_size
    sub = pool8[pages, kv_head, within // 16]                       # [L][sb]
    u = within % 16
    codes = np.take_along_axis(sub, k8_code_offset(u[:, None], np.arange(head_dim)[None, :], head_dim), 1)
    so = k8_scale_offset(u, head_dim)[:, None] + np.arange(4)[None, :]
    scales = np.take_along_axis(sub, so, 1).copy().view(np.float32)[:, 0]
    return codes.view(np.int8).astype(np.float64) * scales.astype(np.float64)[:, None]


def decode_attention_k8(q, pool8, v_pool, block_table, lens, scale, page_size):
    """Decode attention (as ``decode_attention``) over dequantised int8 keys and
    fp16 values. Returns float64 ``[B][Hq][D]``; ``lens[b] == 0`` gives zeros."""
    b_count, hq, d = q.shape
    hkv = v_pool.shape[1]
    g = _check_heads(hq, hkv)
    s64 = _scale64(scale)
    out = np.zeros((b_count, hq, d), dtype=np.float64)
    for b in range(b_count):
        n = int(lens[b])
        if n == 0:
            continue
        for kvh in range(hkv):
            keys = k8_gather_sequence(pool8, block_table[b], n, kvh, page_size, d)
            vals = gather_sequence(v_pool, block_table[b], n, kvh, page_size, "v")
            for i in range(g):
                h = kvh * g + i
                s = s64 * (keys @ q[b, h].astype(np.float64))
                p = np.exp(s - s.max())
                out[b, h] = (p @ vals) / p.sum()
    return out


def decode_attention_multi_k8(q, pool8, v_pool, block_table, lens, scale, page_size):
    """Chunks of queries over int8 keys: ``q`` is ``[B][k][Hq][D]``, query ``i``
    of sequence ``b`` sits at position ``lens[b] - k + i`` and sees tokens
    ``0 .. lens[b] - k + i`` (the reading of chunked attention taken for fp16
    keys in ``decode_attention_multi``), each query computed as the int8-key
    decode step over its own prefix (``decode_attention_k8`` with length
    ``lens[b] - k + i + 1``). Returns float64 ``[B][k][Hq][D]``; a row with
    ``0 < lens[b] < k`` is all NaN; ``lens[b] == 0`` gives zeros."""
    b_count, k, hq, d = q.shape
    out = np.zeros((b_count, k, hq, d), dtype=np.float64)
    lens64 = np.asarray(lens, dtype=np.int64)
    # the chunk would reach before token 0: the whole row is invalid; length 0 is an idle slot (zeros)
    short = (lens64 < k) & (lens64 != 0)
    for i in range(k):
        li = np.where(lens64 < k, 0, lens64 - k + i + 1)
        out[:, i] = decode_attention_k8(q[:, i], pool8, v_pool, block_table, li, scale, page_size)
    out[short] = np.nan
    return out


def decode_attention_window_k8(q, pool8, v_pool, ring_table, lens, window, scale, page_size):
    """Sliding-window decode (the ring of pages of ``decode_attention_window``:
    logical page ``j`` of sequence ``b`` in ``ring_table[b][j % R]``, query ``b``
    attends tokens ``max(0, lens[b] - window) .. lens[b] - 1``) over int8 keys:
    token ``t`` is read as ``code * scale`` from slot ``t % P`` of its ring page.
    Returns float64 ``[B][Hq][D]``; ``lens[b] == 0`` gives zeros."""
    from .paged_decode import _tiles, pool_dims, v_tile_offset
    b_count, hq, d = q.shape
    n, hkv, p, dim = pool_dims(v_pool)
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
        within = t % page_size
        sub = _subblocks(pool8, dim)[pages, :, within // 16]            # [T][Hkv][sb]
        u = within % 16
        for kvh in range(hkv):
            blk = sub[:, kvh]
            codes = np.take_along_axis(blk, k8_code_offset(u[:, None], np.arange(dim)[None, :], dim), 1)
            so = k8_scale_offset(u, dim)[:, None] + np.arange(4)[None, :]
            scales = np.take_along_axis(blk, so, 1).copy().view(np.float32)[:, 0]
            keys = codes.view(np.int8).astype(np.float64) * scales.astype(np.float64)[:, None]
            vals = _tiles(v_pool)[pages[:, None], kvh, v_tile_offset(within[:, None], np.arange(dim)[None, :], p,
                                                                       dim)].astype(np.float64)
            for i in range(g):
                h = kvh * g + i
                sc = s64 * (keys @ q[b, h].astype(np.float64))
                w = np.exp(sc - sc.max())
                out[b, h] = (w @ vals) / w.sum()
    return out


def decode_attention_window_multi_k8(q, pool8, v_pool, ring_table, lens, window, scale, page_size):
    """``decode_attention_window_multi`` over int8 keys: query ``i`` of sequence
    ``b`` is the int8-key window decode step (``decode_attention_window_k8``)
    of its own prefix ``lens[b] - k + i + 1``; a row with ``0 < lens[b] < k``
    is all NaN, ``lens[b] == 0`` gives zeros; ``window + k - 1 <= (R - 1) * P + 1``."""
    b_count, k, hq, d = q.shape
    r = np.asarray(ring_table).shape[1]
    if window + k - 1 > (r - 1) * page_size + 1:
        raise ValueError("the chunk's windows must fit in the ring")
    out = np.zeros((b_count, k, hq, d), dtype=np.float64)
    lens64 = np.asarray(lens, dtype=np.int64)
    short = (lens64 < k) & (lens64 != 0)        # length 0: an idle slot (zeros)
    for i in range(k):
        li = np.where(lens64 < k, 0, lens64 - k + i + 1)
        out[:, i] = decode_attention_window_k8(q[:, i], pool8, v_pool, ring_table, li, window, scale, page_size)
    out[short] = np.nan
    return out


def kv_append_k8(pool8, v_pool, k_new, v_new, block_table, pos, page_size):
    """Copies of the pools with each sequence's new token written: its key
    quantised (``quantize_k``) into the int8 pool, its value as fp16 (the
    in-place append of pgsm §4.3, keys only quantised as dpshk §4.4 advises)."""
    from .paged_decode import write_token
    k_out = pool8.copy()
    v_out = v_pool.copy()
    b_count, hkv, dim = k_new.shape
    for b in range(b_count):
        page, off = token_slot(block_table[b], int(pos[b]), page_size)
        for kvh in range(hkv):
            codes, scale = quantize_k(k_new[b, kvh, :])
            k8_write_token(k_out, page, kvh, off, codes, scale, dim)
            write_token(v_out, page, kvh, off, v_new[b, kvh, :], "v")
    return k_out, v_out
