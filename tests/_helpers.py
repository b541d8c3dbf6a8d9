"""Test-side helpers built on the oracle's data-format functions."""

import numpy as np

import oracle


def poison_unused(w, lens, k_pool=None, v_pool=None, fill=np.nan):
    """Copy of the pools with every slot no sequence attends to set to ``fill``.

    ``lens`` is the per-sequence context that will be attended; slots past it
    in a sequence's last page, and pages no sequence uses, become NaN, so any
    read of them shows in the output.
    """
    k = (w.k_pool if k_pool is None else k_pool).copy()
    v = (w.v_pool if v_pool is None else v_pool).copy()
    live = np.zeros((w.N, w.P), dtype=bool)
    for b in range(w.B):
        n = int(lens[b])
        for j in range(-(-n // w.P)):
            page = int(w.block_table[b, j])
            live[page, :min(w.P, n - j * w.P)] = True
    pages, slots = np.nonzero(~live)
    if len(pages) == 0:
        return k, v
    dims = np.arange(w.D)
    for pool, f in ((k, oracle.k_tile_offset), (v, oracle.v_tile_offset)):
        tiles = pool.reshape(w.N, w.Hkv, w.P * w.D)
        off = f(slots[:, None], dims[None, :], w.P, w.D)
        for kvh in range(w.Hkv):
            tiles[pages[:, None], kvh, off] = fill
    return k, v


def fill_tokens(pool, block_table_row, tokens, values, kind):
    """Write ``values[kvh][i]`` (D halves) as logical tokens ``tokens[i]`` of a
    sequence through its page-table row, in the tile layout of ``kind``."""
    n, hkv, p, d = pool.shape
    tokens = np.asarray(tokens)
    pages = np.asarray(block_table_row)[tokens // p]
    f = oracle.k_tile_offset if kind == "k" else oracle.v_tile_offset
    off = f((tokens % p)[:, None], np.arange(d)[None, :], p, d)
    tiles = pool.reshape(n, hkv, p * d)
    for kvh in range(hkv):
        tiles[pages[:, None], kvh, off] = values[kvh]


def set_dims(pool, block_table_row, token, kvh, dims, value, kind):
    """Set single dims of one token (tile layout of ``kind``)."""
    n, hkv, p, d = pool.shape
    page = int(block_table_row[token // p])
    f = oracle.k_tile_offset if kind == "k" else oracle.v_tile_offset
    pool.reshape(n, hkv, p * d)[page, kvh, f(token % p, np.asarray(dims), p, d)] = value
