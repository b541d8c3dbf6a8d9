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
    n, hkv, p, d = oracle.pool_dims(pool)
    tokens = np.asarray(tokens)
    pages = np.asarray(block_table_row)[tokens // p]
    f = oracle.k_tile_offset if kind == "k" else oracle.v_tile_offset
    off = f((tokens % p)[:, None], np.arange(d)[None, :], p, d)
    tiles = pool.reshape(n, hkv, p * d)
    for kvh in range(hkv):
        tiles[pages[:, None], kvh, off] = values[kvh]


def set_dims(pool, block_table_row, token, kvh, dims, value, kind):
    """Set single dims of one token (tile layout of ``kind``)."""
    n, hkv, p, d = oracle.pool_dims(pool)
    page = int(block_table_row[token // p])
    f = oracle.k_tile_offset if kind == "k" else oracle.v_tile_offset
    pool.reshape(n, hkv, p * d)[page, kvh, f(token % p, np.asarray(dims), p, d)] = value


def poison(pool, live, kind):
    """NaN into every slot of an fp16 pool that `live` [N][P] does not mark."""
    n, hkv, p, d = oracle.pool_dims(pool)
    pages, slots = np.nonzero(~live)
    if len(pages) == 0:
        return pool
    f = oracle.k_tile_offset if kind == "k" else oracle.v_tile_offset
    off = f(slots[:, None], np.arange(d)[None, :], p, d)
    tiles = pool.reshape(n, hkv, p * d)
    for kvh in range(hkv):
        tiles[pages[:, None], kvh, off] = np.nan
    return pool


def live_slots(N, P, table, lens, lo=None):
    """[N][P] mask of the slots holding tokens [lo[b], lens[b]) of each row
    (table columns taken modulo the table width, as a ring does)."""
    live = np.zeros((N, P), dtype=bool)
    R = table.shape[1]
    for b in range(table.shape[0]):
        start = 0 if lo is None else int(lo[b])
        t = np.arange(start, max(int(lens[b]), start))
        if len(t):
            live[table[b, (t // P) % R], t % P] = True
    return live


def k8_pool(rng, N, Hkv, P, D, live):
    codes = rng.integers(-127, 128, size=(N, Hkv, P // 16, 16 * D)).astype(np.int8).view(np.uint8)
    scales = (np.abs(rng.standard_normal((N, Hkv, P // 16, 16))) * 0.05 + 0.005).astype(np.float32)
    dead = ~live.reshape(N, 1, P // 16, 16)
    scales = np.where(np.broadcast_to(dead, scales.shape), np.float32(np.nan), scales)
    return np.ascontiguousarray(np.concatenate([codes, scales.view(np.uint8)], axis=-1))
