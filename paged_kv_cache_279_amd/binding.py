"""ctypes binding over libpkv.so: argument marshalling only.

Every function mirrors the C entry point of the same name in ``include/pkv.h``
(without the ``pkv_`` prefix). Tensors are torch tensors: device tensors for
the device entry points, host int32 arrays (numpy or torch) for the allocator.
torch is used for device memory and streams; all arithmetic of the decode path
runs in the library's HIP kernels. There is no fallback: if ``libpkv.so`` is
missing or fails to load, every call raises.
"""

import ctypes
import os

import numpy as np
import torch  # loaded before libpkv.so so both share torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = 1
PKV_ERR_UNSUPPORTED = 2
PKV_ERR_OUT_OF_PAGES = 3
PKV_ERR_WORKSPACE_TOO_SMALL = 4
PKV_ERR_HIP = 5
PKV_ERR_INVALID_TABLE = 6
PKV_ERR_NOT_FOUND = 7
PKV_ERR_HOST_MEMORY = 8
PKV_ERR_SCRATCH_LIMIT = 9

_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_ip = ctypes.POINTER(ctypes.c_int32)

_SIGNATURES = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_abi_version": (ctypes.c_int, []),
    "pkv_kv_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pkv_kv_append_chunk": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                            _vp]),
    "pkv_block_table_patch": (ctypes.c_int, [_vp, _i32, _i32, _ip, _ip, _ip, _i32, _vp]),
    "pkv_probe_stream_read": (ctypes.c_int, [_vp, ctypes.c_size_t, _vp, _i32, _i32, _vp, _vp]),
    "pkv_profile_next_partition_kernel": (ctypes.c_int, [_vp, _vp]),
    "pkv_k8_pool_bytes": (ctypes.c_int, [_i32, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]),
    "pkv_paged_decode_attention_multi": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                                        _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _vp,
                                                        ctypes.c_size_t, _vp]),
    "pkv_paged_decode_attention_window": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                                         _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _vp,
                                                         ctypes.c_size_t, _vp]),
    "pkv_paged_decode_attention_multi_shared_prefix": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                                                      _i32, _i32, _i32, _i32, _i32, _i32,
                                                                      ctypes.c_float, _i32, _i32, _vp,
                                                                      ctypes.c_size_t, _vp]),
    "pkv_kv_append_k8_chunk": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                               _vp]),
    "pkv_paged_decode_attention_multi_k8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                                           _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _i32, _vp,
                                                           ctypes.c_size_t, _vp]),
    "pkv_paged_decode_attention_window_k8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                                            _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _vp,
                                                            ctypes.c_size_t, _vp]),
    "pkv_paged_decode_attention_window_multi": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _vp, ctypes.c_size_t, _vp]),
    "pkv_paged_decode_attention_window_multi_k8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _vp, ctypes.c_size_t, _vp]),
    "pkv_kv_append_k8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pkv_paged_decode_attention_k8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                                     _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _i32, _vp,
                                                     ctypes.c_size_t, _vp]),
    "pkv_decode_workspace_bytes": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]),
    "pkv_paged_decode_attention": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                                  _i32, _i32, ctypes.c_float, _i32, _vp, ctypes.c_size_t, _vp]),
    "pkv_append_paged_decode_attention": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                                         _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _vp,
                                                         ctypes.c_size_t, _vp]),
    "pkv_decode_workspace_bytes_shared_prefix": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32,
                                                                 ctypes.POINTER(ctypes.c_size_t)]),
    "pkv_decode_workspace_bytes_multi": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                         ctypes.POINTER(ctypes.c_size_t)]),
    "pkv_paged_decode_attention_shared_prefix": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                                                _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_float,
                                                                _i32, _i32, _vp, ctypes.c_size_t, _vp]),
    "pkv_paged_decode_attention_shared_prefix_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                                                        _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                                        ctypes.c_float, _i32, _i32, _vp]),
    "pkv_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "pkv_alloc_create": (ctypes.c_int, [_i32, _i32, _ip, ctypes.POINTER(_vp)]),
    "pkv_alloc_destroy": (None, [_vp]),
    "pkv_alloc_reserve": (ctypes.c_int, [_vp, _i32, _i32, _ip, _i32, _ip]),
    "pkv_alloc_reserve_batch": (ctypes.c_int, [_vp, _i32, _ip, _ip, _ip, _i32]),
    "pkv_alloc_share_prefix": (ctypes.c_int, [_vp, _i32, _ip, _i32]),
    "pkv_alloc_free": (ctypes.c_int, [_vp, _i32]),
    "pkv_alloc_free_count": (ctypes.c_int32, [_vp]),
    "pkv_alloc_table": (ctypes.c_int, [_vp, _i32, _ip, _i32, _ip]),
    "pkv_alloc_refcount": (ctypes.c_int, [_vp, _i32, _ip]),
    "pkv_alloc_cache_insert": (ctypes.c_int, [_vp, ctypes.c_uint64, _i32, _i32]),
    "pkv_alloc_cache_lookup": (ctypes.c_int, [_vp, ctypes.c_uint64, _ip, _i32, _ip, _ip]),
    "pkv_alloc_cache_evict": (ctypes.c_int, [_vp, ctypes.c_uint64]),
    "pkv_alloc_cache_entries": (ctypes.c_int32, [_vp]),
    "pkv_alloc_prepare_append": (ctypes.c_int, [_vp, _i32, _ip, _ip, _ip, _ip, _ip, _ip, _i32]),
    "pkv_copy_pages": (ctypes.c_int, [_vp, ctypes.c_size_t, _i32, _ip, _ip, _i32, _vp]),
    "pkv_validate_tables": (ctypes.c_int, [_ip, _ip, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _ip, _ip, _ip]),
}

_LIB = None


class PkvError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, status_string(status)))


def lib():
    """Load libpkv.so once; raise if it is not built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpkv.so is not built; run `python -m paged_kv_cache_279_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def status_string(status):
    return lib().pkv_status_string(int(status)).decode()


def _check(status, where):
    if status != PKV_OK:
        raise PkvError(status, where)


def _dev_ptr(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %d" % (name, ndim, t.dim()))
    return ctypes.c_void_p(t.data_ptr())


def pool_shape(N, Hkv, P, D):
    """Storage shape of an fp16 K or V pool: N pages x Hkv KV heads x P/16
    sub-blocks of 16 tokens x 16*D halves. A sub-block is in the library's
    matrix-core operand order (``include/pkv.h``), not [token][dim]: write
    tokens with kv_append, never by indexing."""
    if P % 16 or P <= 0 or D <= 0:
        raise ValueError("P must be a positive multiple of 16")
    return (N, Hkv, P // 16, 16 * D)


def empty_pool(N, Hkv, P, D, device="cuda"):
    """An uninitialised fp16 pool of ``pool_shape(N, Hkv, P, D)`` on ``device``."""
    return torch.empty(pool_shape(N, Hkv, P, D), dtype=torch.float16, device=device)


def _f16_pool(pool, name, head_dim):
    """(N, Hkv, P, D) of an fp16 pool tensor of storage shape [N][Hkv][P/16][16*D],
    D = ``head_dim`` (taken from the queries or new tokens)."""
    if not isinstance(pool, torch.Tensor) or pool.dim() != 4 or pool.dtype != torch.float16 or \
            pool.shape[3] != 16 * head_dim:
        raise ValueError("%s must be an fp16 pool of storage shape [N][Hkv][P/16][16*D] (pool_shape), D = %d; got %s"
                         % (name, head_dim, tuple(pool.shape) if isinstance(pool, torch.Tensor) else type(pool)))
    N, Hkv, nsub, w = pool.shape
    return N, Hkv, 16 * nsub, w // 16


def _workspace_arg(workspace, ws_bytes, device):
    """Pointer and byte size of the split-mode workspace: the caller's (a
    contiguous device tensor of any dtype; the library checks the size), or a
    new one of ``ws_bytes`` bytes; NULL and 0 when none is needed or given."""
    if workspace is None:
        if ws_bytes == 0:
            return ctypes.c_void_p(0), 0
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ---------------------------------------------------------------------------
# device entry points
# ---------------------------------------------------------------------------

def block_table_patch(block_table, rows, cols, pages, stream=None):
    """pkv_block_table_patch: block_table[rows[i], cols[i]] = pages[i] on the device (host lists)."""
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B][max_pages]")
    B, max_pages = block_table.shape
    r, rp = _host_i32(rows, "rows")
    c, cp = _host_i32(cols, "cols")
    g, gp = _host_i32(pages, "pages")
    if not (r.shape == c.shape == g.shape) or r.ndim != 1:
        raise ValueError("rows, cols and pages must be 1-D and of one length")
    _check(lib().pkv_block_table_patch(_dev_ptr(block_table, torch.int32, "block_table"), B, max_pages, rp, cp, gp,
                                       len(r), _stream(stream)), "pkv_block_table_patch")
    return block_table


def probe_stream_read(buf, tile_order, sink, waves=8192, stream=None):
    """pkv_probe_stream_read: read the 4 KiB tiles of ``buf`` (a uint8 device
    tensor) in ``tile_order`` (int32 device) -- the streaming-read ceiling."""
    if buf.dtype != torch.uint8 or tile_order.dtype != torch.int32 or tile_order.dim() != 1:
        raise ValueError("buf must be uint8, tile_order 1-D int32")
    _check(lib().pkv_probe_stream_read(_dev_ptr(buf, torch.uint8, "buf"), buf.numel(),
                                       _dev_ptr(tile_order, torch.int32, "tile_order"), tile_order.numel(),
                                       int(waves), _dev_ptr(sink, torch.int32, "sink"), _stream(stream)),
           "pkv_probe_stream_read")


def profile_next_partition_kernel(start, stop):
    """pkv_profile_next_partition_kernel: the next decode call on this thread records
    its partition kernel's start and stop into ``start`` / ``stop``
    (torch.cuda.Event(enable_timing=True), each recorded once before so that it exists)."""
    handles = []
    for ev in (start, stop):
        h = int(getattr(ev, "cuda_event", 0) or 0)
        if h == 0:
            raise ValueError("record the event once first: torch creates it on its first record")
        handles.append(ctypes.c_void_p(h))
    _check(lib().pkv_profile_next_partition_kernel(*handles), "pkv_profile_next_partition_kernel")


def copy_pages(pool, src, dst, stream=None):
    """pkv_copy_pages: page dst[i] of ``pool`` (a device tensor whose first axis is the
    page) becomes a copy of page src[i]."""
    s, sp = _host_i32(src, "src")
    d, dp = _host_i32(dst, "dst")
    if s.shape != d.shape:
        raise ValueError("src and dst must have one length")
    if not pool.is_cuda or not pool.is_contiguous():
        raise ValueError("pool must be a contiguous device tensor")
    page_bytes = pool[0].numel() * pool.element_size()
    _check(lib().pkv_copy_pages(ctypes.c_void_p(pool.data_ptr()), page_bytes, pool.shape[0], sp, dp, len(s),
                                _stream(stream)), "pkv_copy_pages")


def kv_append(k_new, v_new, k_pool, v_pool, block_table, pos, stream=None):
    """pkv_kv_append: write k_new/v_new [B][Hkv][D] at slot pos[b] of each sequence."""
    N, Hkv, P, D = _f16_pool(k_pool, "k_pool", int(k_new.shape[-1]))
    B, max_pages = block_table.shape
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("shape mismatch")
    if tuple(pos.shape) != (B,):
        raise ValueError("pos must be [B]")
    rc = lib().pkv_kv_append(_dev_ptr(k_new, torch.float16, "k_new"), _dev_ptr(v_new, torch.float16, "v_new"),
                             _dev_ptr(k_pool, torch.float16, "k_pool"), _dev_ptr(v_pool, torch.float16, "v_pool"),
                             _dev_ptr(block_table, torch.int32, "block_table"), max_pages,
                             _dev_ptr(pos, torch.int32, "pos"), B, Hkv, D, P, N, _stream(stream))
    _check(rc, "pkv_kv_append")


def kv_append_chunk(k_new, v_new, k_pool, v_pool, block_table, pos, stream=None):
    """pkv_kv_append_chunk: write k_new/v_new [B][n_tokens][Hkv][D]; token i of sequence b
    goes to position pos[b] + i."""
    N, Hkv, P, D = _f16_pool(k_pool, "k_pool", int(k_new.shape[-1]))
    B, max_pages = block_table.shape
    if k_new.dim() != 4 or tuple(k_new.shape) != tuple(v_new.shape) or k_new.shape[0] != B or \
            tuple(k_new.shape[2:]) != (Hkv, D) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_new/v_new must be [B][n_tokens][Hkv][D] matching the pools and the table")
    if tuple(pos.shape) != (B,):
        raise ValueError("pos must be [B]")
    rc = lib().pkv_kv_append_chunk(_dev_ptr(k_new, torch.float16, "k_new"), _dev_ptr(v_new, torch.float16, "v_new"),
                                   _dev_ptr(k_pool, torch.float16, "k_pool"), _dev_ptr(v_pool, torch.float16, "v_pool"),
                                   _dev_ptr(block_table, torch.int32, "block_table"), max_pages,
                                   _dev_ptr(pos, torch.int32, "pos"), B, int(k_new.shape[1]), Hkv, D, P, N,
                                   _stream(stream))
    _check(rc, "pkv_kv_append_chunk")


def paged_decode_attention_shared_prefix_noalloc(q, k_pool, v_pool, block_table, lens, max_context, scale,
                                                 partition_tokens, prefix_tokens, out, k_new=None, v_new=None,
                                                 stream=None):
    """pkv_paged_decode_attention_shared_prefix_noalloc: the shared-prefix call with the split
    partials in the library's fixed scratch array; ``out`` (fp16 [B][Hq][D]) must be given --
    nothing is allocated."""
    B, Hq, D = q.shape
    N, Hkv, P, _ = _f16_pool(k_pool, "k_pool", int(D))
    _, max_pages = block_table.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape) or block_table.shape[0] != B or tuple(lens.shape) != (B,):
        raise ValueError("shape mismatch")
    if out is None or tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be given, [B][Hq][D]")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
            raise ValueError("k_new/v_new must be [B][Hkv][D]")
        kn, vn = _dev_ptr(k_new, torch.float16, "k_new"), _dev_ptr(v_new, torch.float16, "v_new")
    else:
        kn, vn = ctypes.c_void_p(0), ctypes.c_void_p(0)
    rc = lib().pkv_paged_decode_attention_shared_prefix_noalloc(
        _dev_ptr(out, torch.float16, "out"), _dev_ptr(q, torch.float16, "q"), kn, vn,
        _dev_ptr(k_pool, torch.float16, "k_pool"), _dev_ptr(v_pool, torch.float16, "v_pool"),
        _dev_ptr(block_table, torch.int32, "block_table"), max_pages, _dev_ptr(lens, torch.int32, "lens"),
        B, Hq, Hkv, D, P, N, int(max_context), float(scale), int(partition_tokens), int(prefix_tokens),
        _stream(stream))
    _check(rc, "pkv_paged_decode_attention_shared_prefix_noalloc")
    return out


def noalloc_scratch_bytes():
    """pkv_noalloc_scratch_bytes: size of the no-allocation entry point's fixed scratch array."""
    return int(lib().pkv_noalloc_scratch_bytes())


def paged_decode_attention_multi(q, k_pool, v_pool, block_table, lens, max_context, scale, partition_tokens=0,
                                 out=None, workspace=None, stream=None, prefix_tokens=0):
    """pkv_paged_decode_attention_multi: q [B][n_query][Hq][D], the last n_query tokens of
    each sequence, causal within the chunk; returns ``out`` [B][n_query][Hq][D]. With
    prefix_tokens > 0 the batch shares its first prefix_tokens tokens
    (pkv_paged_decode_attention_multi_shared_prefix)."""
    B, nq, Hq, D = q.shape
    N, Hkv, P, Dk = _f16_pool(k_pool, "k_pool", int(q.shape[-1]))
    _, max_pages = block_table.shape
    if Dk != D or tuple(v_pool.shape) != tuple(k_pool.shape) or block_table.shape[0] != B or tuple(lens.shape) != (B,):
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((B, nq, Hq, D), dtype=torch.float16, device=q.device)
    if tuple(out.shape) != (B, nq, Hq, D):
        raise ValueError("out must be [B][n_query][Hq][D]")
    ws_bytes = decode_workspace_bytes_multi(B, nq, Hq, D, max_context, partition_tokens, prefix_tokens)
    ws_ptr, ws_len = _workspace_arg(workspace, ws_bytes, q.device)
    ptrs = (_dev_ptr(out, torch.float16, "out"), _dev_ptr(q, torch.float16, "q"),
            _dev_ptr(k_pool, torch.float16, "k_pool"), _dev_ptr(v_pool, torch.float16, "v_pool"),
            _dev_ptr(block_table, torch.int32, "block_table"), max_pages, _dev_ptr(lens, torch.int32, "lens"),
            B, nq, Hq, Hkv, D, P, N, int(max_context), float(scale), int(partition_tokens))
    if prefix_tokens:
        rc = lib().pkv_paged_decode_attention_multi_shared_prefix(*ptrs, int(prefix_tokens), ws_ptr, ws_len,
                                                                  _stream(stream))
        _check(rc, "pkv_paged_decode_attention_multi_shared_prefix")
    else:
        rc = lib().pkv_paged_decode_attention_multi(*ptrs, ws_ptr, ws_len, _stream(stream))
        _check(rc, "pkv_paged_decode_attention_multi")
    return out


def paged_decode_attention_window(q, k_pool, v_pool, ring_table, lens, window, scale, partition_tokens=0,
                                  k_new=None, v_new=None, out=None, workspace=None, stream=None):
    """pkv_paged_decode_attention_window: attend the last ``window`` tokens of each sequence,
    logical page j in ``ring_table[b][j % ring_pages]``; with k_new / v_new the new token is
    appended at lens[b] - 1 in the same launch. Returns ``out`` [B][Hq][D]."""
    B, Hq, D = q.shape
    N, Hkv, P, Dk = _f16_pool(k_pool, "k_pool", int(q.shape[-1]))
    _, ring_pages = ring_table.shape
    if Dk != D or tuple(v_pool.shape) != tuple(k_pool.shape) or ring_table.shape[0] != B or tuple(lens.shape) != (B,):
        raise ValueError("shape mismatch")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None and (tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D)):
        raise ValueError("k_new / v_new must be [B][Hkv][D]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=q.device)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B][Hq][D]")
    ws_bytes = decode_workspace_bytes(B, Hq, D, int(window), partition_tokens)
    ws_ptr, ws_len = _workspace_arg(workspace, ws_bytes, q.device)
    kn = _dev_ptr(k_new, torch.float16, "k_new") if k_new is not None else ctypes.c_void_p(0)
    vn = _dev_ptr(v_new, torch.float16, "v_new") if v_new is not None else ctypes.c_void_p(0)
    rc = lib().pkv_paged_decode_attention_window(
        _dev_ptr(out, torch.float16, "out"), _dev_ptr(q, torch.float16, "q"), kn, vn,
        _dev_ptr(k_pool, torch.float16, "k_pool"), _dev_ptr(v_pool, torch.float16, "v_pool"),
        _dev_ptr(ring_table, torch.int32, "ring_table"), ring_pages, _dev_ptr(lens, torch.int32, "lens"),
        B, Hq, Hkv, D, P, N, int(window), float(scale), int(partition_tokens), ws_ptr, ws_len, _stream(stream))
    _check(rc, "pkv_paged_decode_attention_window")
    return out


def paged_decode_attention_window_multi(q, k_pool, v_pool, ring_table, lens, window, scale, partition_tokens=0,
                                        out=None, workspace=None, stream=None):
    """pkv_paged_decode_attention_window_multi (fp16 keys) or, when ``k_pool`` is an int8-key pool
    (uint8 [N][Hkv][P/16][16 D + 64]), pkv_paged_decode_attention_window_multi_k8: chunks of
    queries q [B][n_query][Hq][D], each attending the window ending at itself through the ring."""
    k8 = k_pool.dtype == torch.uint8
    if k8:
        N, Hkv, P, D = _k8_shape(k_pool, v_pool, int(q.shape[-1]))
    else:
        N, Hkv, P, D = _f16_pool(k_pool, "k_pool", int(q.shape[-1]))
        if tuple(v_pool.shape) != tuple(k_pool.shape):
            raise ValueError("shape mismatch")
    B, nq, Hq, Dq = q.shape
    _, ring_pages = ring_table.shape
    if Dq != D or ring_table.shape[0] != B or tuple(lens.shape) != (B,):
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((B, nq, Hq, D), dtype=torch.float16, device=q.device)
    if tuple(out.shape) != (B, nq, Hq, D):
        raise ValueError("out must be [B][n_query][Hq][D]")
    ws_ptr, ws_len = _workspace_arg(workspace, decode_workspace_bytes_multi(B, nq, Hq, D, int(window),
                                                                            partition_tokens), q.device)
    fn = lib().pkv_paged_decode_attention_window_multi_k8 if k8 else lib().pkv_paged_decode_attention_window_multi
    rc = fn(_dev_ptr(out, torch.float16, "out"), _dev_ptr(q, torch.float16, "q"),
            _dev_ptr(k_pool, torch.uint8 if k8 else torch.float16, "k_pool"), _dev_ptr(v_pool, torch.float16, "v_pool"),
            _dev_ptr(ring_table, torch.int32, "ring_table"), ring_pages, _dev_ptr(lens, torch.int32, "lens"),
            B, nq, Hq, Hkv, D, P, N, int(window), float(scale), int(partition_tokens), ws_ptr, ws_len,
            _stream(stream))
    _check(rc, "pkv_paged_decode_attention_window_multi" + ("_k8" if k8 else ""))
    return out


def k8_pool_bytes(N, Hkv, P, D):
    """pkv_k8_pool_bytes: bytes of an int8-key pool [N][Hkv][P/16][16 D + 64]."""
    out = ctypes.c_size_t(0)
    _check(lib().pkv_k8_pool_bytes(N, Hkv, P, D, ctypes.byref(out)), "pkv_k8_pool_bytes")
    return out.value


def _k8_shape(k_pool8, v_pool, head_dim):
    N, Hkv, P, D = _f16_pool(v_pool, "v_pool", head_dim)
    if k_pool8.dtype != torch.uint8 or tuple(k_pool8.shape) != (N, Hkv, P // 16, 16 * D + 64):
        raise ValueError("k_pool8 must be uint8 [N][Hkv][P/16][16 D + 64] matching v_pool [N][Hkv][P/16][16 D]")
    return N, Hkv, P, D


def kv_append_k8(k_new, v_new, k_pool8, v_pool, block_table, pos, stream=None):
    """pkv_kv_append_k8: quantise k_new into the int8-key pool, write v_new into the fp16 V pool."""
    N, Hkv, P, D = _k8_shape(k_pool8, v_pool, int(k_new.shape[-1]))
    B, max_pages = block_table.shape
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D) or tuple(pos.shape) != (B,):
        raise ValueError("shape mismatch")
    _check(lib().pkv_kv_append_k8(_dev_ptr(k_new, torch.float16, "k_new"), _dev_ptr(v_new, torch.float16, "v_new"),
                                  _dev_ptr(k_pool8, torch.uint8, "k_pool8"), _dev_ptr(v_pool, torch.float16, "v_pool"),
                                  _dev_ptr(block_table, torch.int32, "block_table"), max_pages,
                                  _dev_ptr(pos, torch.int32, "pos"), B, Hkv, D, P, N, _stream(stream)),
           "pkv_kv_append_k8")


def kv_append_k8_chunk(k_new, v_new, k_pool8, v_pool, block_table, pos, stream=None):
    """pkv_kv_append_k8_chunk: k_new/v_new [B][n_tokens][Hkv][D]; token i of sequence b goes to
    position pos[b] + i, its key quantised into the int8-key pool."""
    N, Hkv, P, D = _k8_shape(k_pool8, v_pool, int(k_new.shape[-1]))
    B, max_pages = block_table.shape
    if k_new.dim() != 4 or tuple(k_new.shape) != tuple(v_new.shape) or k_new.shape[0] != B or \
            tuple(k_new.shape[2:]) != (Hkv, D) or tuple(pos.shape) != (B,):
        raise ValueError("k_new/v_new must be [B][n_tokens][Hkv][D], pos [B]")
    _check(lib().pkv_kv_append_k8_chunk(_dev_ptr(k_new, torch.float16, "k_new"),
                                        _dev_ptr(v_new, torch.float16, "v_new"),
                                        _dev_ptr(k_pool8, torch.uint8, "k_pool8"),
                                        _dev_ptr(v_pool, torch.float16, "v_pool"),
                                        _dev_ptr(block_table, torch.int32, "block_table"), max_pages,
                                        _dev_ptr(pos, torch.int32, "pos"), B, int(k_new.shape[1]), Hkv, D, P, N,
                                        _stream(stream)), "pkv_kv_append_k8_chunk")


def paged_decode_attention_multi_k8(q, k_pool8, v_pool, block_table, lens, max_context, scale, partition_tokens=0,
                                    prefix_tokens=0, out=None, workspace=None, stream=None):
    """pkv_paged_decode_attention_multi_k8: chunks of queries q [B][n_query][Hq][D] over int8
    keys and fp16 values; returns ``out`` [B][n_query][Hq][D]."""
    N, Hkv, P, D = _k8_shape(k_pool8, v_pool, int(q.shape[-1]))
    B, nq, Hq, Dq = q.shape
    _, max_pages = block_table.shape
    if Dq != D or block_table.shape[0] != B or tuple(lens.shape) != (B,):
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((B, nq, Hq, D), dtype=torch.float16, device=q.device)
    if tuple(out.shape) != (B, nq, Hq, D):
        raise ValueError("out must be [B][n_query][Hq][D]")
    ws_bytes = decode_workspace_bytes_multi(B, nq, Hq, D, max_context, partition_tokens, prefix_tokens)
    ws_ptr, ws_len = _workspace_arg(workspace, ws_bytes, q.device)
    rc = lib().pkv_paged_decode_attention_multi_k8(
        _dev_ptr(out, torch.float16, "out"), _dev_ptr(q, torch.float16, "q"), _dev_ptr(k_pool8, torch.uint8, "k_pool8"),
        _dev_ptr(v_pool, torch.float16, "v_pool"), _dev_ptr(block_table, torch.int32, "block_table"), max_pages,
        _dev_ptr(lens, torch.int32, "lens"), B, nq, Hq, Hkv, D, P, N, int(max_context), float(scale),
        int(partition_tokens), int(prefix_tokens), ws_ptr, ws_len, _stream(stream))
    _check(rc, "pkv_paged_decode_attention_multi_k8")
    return out


def paged_decode_attention_window_k8(q, k_pool8, v_pool, ring_table, lens, window, scale, partition_tokens=0,
                                     k_new=None, v_new=None, out=None, workspace=None, stream=None):
    """pkv_paged_decode_attention_window_k8: the sliding-window call over an int8-key pool
    (logical page j in ring_table[b][j % ring_pages]); optional fused quantising append."""
    N, Hkv, P, D = _k8_shape(k_pool8, v_pool, int(q.shape[-1]))
    B, Hq, Dq = q.shape
    _, ring_pages = ring_table.shape
    if Dq != D or ring_table.shape[0] != B or tuple(lens.shape) != (B,):
        raise ValueError("shape mismatch")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None and (tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D)):
        raise ValueError("k_new / v_new must be [B][Hkv][D]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=q.device)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B][Hq][D]")
    ws_ptr, ws_len = _workspace_arg(workspace, decode_workspace_bytes(B, Hq, D, int(window), partition_tokens),
                                    q.device)
    kn = _dev_ptr(k_new, torch.float16, "k_new") if k_new is not None else ctypes.c_void_p(0)
    vn = _dev_ptr(v_new, torch.float16, "v_new") if v_new is not None else ctypes.c_void_p(0)
    rc = lib().pkv_paged_decode_attention_window_k8(
        _dev_ptr(out, torch.float16, "out"), _dev_ptr(q, torch.float16, "q"), kn, vn,
        _dev_ptr(k_pool8, torch.uint8, "k_pool8"), _dev_ptr(v_pool, torch.float16, "v_pool"),
        _dev_ptr(ring_table, torch.int32, "ring_table"), ring_pages, _dev_ptr(lens, torch.int32, "lens"),
        B, Hq, Hkv, D, P, N, int(window), float(scale), int(partition_tokens), ws_ptr, ws_len, _stream(stream))
    _check(rc, "pkv_paged_decode_attention_window_k8")
    return out


def paged_decode_attention_k8(q, k_pool8, v_pool, block_table, lens, max_context, scale, partition_tokens=0,
                              prefix_tokens=0, k_new=None, v_new=None, out=None, workspace=None, stream=None):
    """pkv_paged_decode_attention_k8: decode over int8 keys and fp16 values, with the
    new token appended (and its key quantised) first when k_new/v_new are given; returns ``out``."""
    N, Hkv, P, D = _k8_shape(k_pool8, v_pool, int(q.shape[-1]))
    out, (_, _, _, _, B, Hq, max_pages), ws_ptr, ws_len = _decode_args(
        out, q, v_pool, v_pool, block_table, lens, max_context, partition_tokens, workspace, prefix_tokens)
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
            raise ValueError("k_new/v_new must be [B][Hkv][D]")
        kn, vn = _dev_ptr(k_new, torch.float16, "k_new"), _dev_ptr(v_new, torch.float16, "v_new")
    else:
        kn, vn = ctypes.c_void_p(0), ctypes.c_void_p(0)
    rc = lib().pkv_paged_decode_attention_k8(
        _dev_ptr(out, torch.float16, "out"), _dev_ptr(q, torch.float16, "q"), kn, vn,
        _dev_ptr(k_pool8, torch.uint8, "k_pool8"),
        _dev_ptr(v_pool, torch.float16, "v_pool"), _dev_ptr(block_table, torch.int32, "block_table"), max_pages,
        _dev_ptr(lens, torch.int32, "lens"), B, Hq, Hkv, D, P, N, int(max_context), float(scale),
        int(partition_tokens), int(prefix_tokens), ws_ptr, ws_len, _stream(stream))
    _check(rc, "pkv_paged_decode_attention_k8")
    return out


def decode_workspace_bytes(B, Hq, D, max_context, partition_tokens, prefix_tokens=0):
    """pkv_decode_workspace_bytes (or the shared-prefix variant when prefix_tokens > 0)."""
    out = ctypes.c_size_t(0)
    if prefix_tokens:
        rc = lib().pkv_decode_workspace_bytes_shared_prefix(B, Hq, D, max_context, partition_tokens, prefix_tokens,
                                                            ctypes.byref(out))
    else:
        rc = lib().pkv_decode_workspace_bytes(B, Hq, D, max_context, partition_tokens, ctypes.byref(out))
    _check(rc, "pkv_decode_workspace_bytes")
    return out.value


def decode_workspace_bytes_multi(B, n_query, Hq, D, max_context, partition_tokens, prefix_tokens=0):
    """pkv_decode_workspace_bytes_multi: workspace of the chunked calls (n_query queries per sequence)."""
    out = ctypes.c_size_t(0)
    _check(lib().pkv_decode_workspace_bytes_multi(B, n_query, Hq, D, max_context, partition_tokens, prefix_tokens,
                                                  ctypes.byref(out)), "pkv_decode_workspace_bytes_multi")
    return out.value


def _decode_args(out, q, k_pool, v_pool, block_table, lens, max_context, partition_tokens, workspace,
                 prefix_tokens=0):
    N, Hkv, P, D = _f16_pool(k_pool, "k_pool", int(q.shape[-1]))
    B, Hq, Dq = q.shape
    _, max_pages = block_table.shape
    if Dq != D or tuple(v_pool.shape) != tuple(k_pool.shape) or block_table.shape[0] != B or tuple(lens.shape) != (B,):
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=q.device)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B][Hq][D]")
    ws_bytes = decode_workspace_bytes(B, Hq, D, max_context, partition_tokens, prefix_tokens)
    ws_ptr, ws_len = _workspace_arg(workspace, ws_bytes, q.device)
    return out, (N, Hkv, P, D, B, Hq, max_pages), ws_ptr, ws_len


def paged_decode_attention(q, k_pool, v_pool, block_table, lens, max_context, scale, partition_tokens=0,
                           out=None, workspace=None, stream=None):
    """pkv_paged_decode_attention; returns ``out`` (fp16 [B][Hq][D])."""
    out, (N, Hkv, P, D, B, Hq, max_pages), ws_ptr, ws_len = _decode_args(
        out, q, k_pool, v_pool, block_table, lens, max_context, partition_tokens, workspace)
    rc = lib().pkv_paged_decode_attention(
        _dev_ptr(out, torch.float16, "out"), _dev_ptr(q, torch.float16, "q"),
        _dev_ptr(k_pool, torch.float16, "k_pool"), _dev_ptr(v_pool, torch.float16, "v_pool"),
        _dev_ptr(block_table, torch.int32, "block_table"), max_pages, _dev_ptr(lens, torch.int32, "lens"),
        B, Hq, Hkv, D, P, N, int(max_context), float(scale), int(partition_tokens), ws_ptr, ws_len, _stream(stream))
    _check(rc, "pkv_paged_decode_attention")
    return out


def append_paged_decode_attention(q, k_new, v_new, k_pool, v_pool, block_table, lens, max_context, scale,
                                  partition_tokens=0, out=None, workspace=None, stream=None):
    """pkv_append_paged_decode_attention: append at lens-1, then attend; returns ``out``."""
    out, (N, Hkv, P, D, B, Hq, max_pages), ws_ptr, ws_len = _decode_args(
        out, q, k_pool, v_pool, block_table, lens, max_context, partition_tokens, workspace)
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new/v_new must be [B][Hkv][D]")
    rc = lib().pkv_append_paged_decode_attention(
        _dev_ptr(out, torch.float16, "out"), _dev_ptr(q, torch.float16, "q"),
        _dev_ptr(k_new, torch.float16, "k_new"), _dev_ptr(v_new, torch.float16, "v_new"),
        _dev_ptr(k_pool, torch.float16, "k_pool"), _dev_ptr(v_pool, torch.float16, "v_pool"),
        _dev_ptr(block_table, torch.int32, "block_table"), max_pages, _dev_ptr(lens, torch.int32, "lens"),
        B, Hq, Hkv, D, P, N, int(max_context), float(scale), int(partition_tokens), ws_ptr, ws_len, _stream(stream))
    _check(rc, "pkv_append_paged_decode_attention")
    return out


def paged_decode_attention_shared_prefix(q, k_pool, v_pool, block_table, lens, max_context, scale,
                                         partition_tokens, prefix_tokens, k_new=None, v_new=None, out=None,
                                         workspace=None, stream=None):
    """pkv_paged_decode_attention_shared_prefix: every sequence starts with the
    same ``prefix_tokens`` tokens in the same pages; optional fused append."""
    out, (N, Hkv, P, D, B, Hq, max_pages), ws_ptr, ws_len = _decode_args(
        out, q, k_pool, v_pool, block_table, lens, max_context, partition_tokens, workspace, prefix_tokens)
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
            raise ValueError("k_new/v_new must be [B][Hkv][D]")
        kn, vn = _dev_ptr(k_new, torch.float16, "k_new"), _dev_ptr(v_new, torch.float16, "v_new")
    else:
        kn, vn = ctypes.c_void_p(0), ctypes.c_void_p(0)
    rc = lib().pkv_paged_decode_attention_shared_prefix(
        _dev_ptr(out, torch.float16, "out"), _dev_ptr(q, torch.float16, "q"), kn, vn,
        _dev_ptr(k_pool, torch.float16, "k_pool"), _dev_ptr(v_pool, torch.float16, "v_pool"),
        _dev_ptr(block_table, torch.int32, "block_table"), max_pages, _dev_ptr(lens, torch.int32, "lens"),
        B, Hq, Hkv, D, P, N, int(max_context), float(scale), int(partition_tokens), int(prefix_tokens),
        ws_ptr, ws_len, _stream(stream))
    _check(rc, "pkv_paged_decode_attention_shared_prefix")
    return out


# ---------------------------------------------------------------------------
# host allocator
# ---------------------------------------------------------------------------

def _host_i32(a, name):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(_ip)


class PageAllocator:
    """Host page allocator (pkv_alloc_*): FIFO free list, all-or-nothing
    reservations, reference-counted shared prefixes."""

    def __init__(self, num_pages, page_size, free_order=None):
        self._h = ctypes.c_void_p(0)
        if free_order is None:
            rc = lib().pkv_alloc_create(num_pages, page_size, None, ctypes.byref(self._h))
        else:
            arr, ptr = _host_i32(free_order, "free_order")
            if arr.shape != (num_pages,):
                raise ValueError("free_order must have num_pages entries")
            rc = lib().pkv_alloc_create(num_pages, page_size, ptr, ctypes.byref(self._h))
        _check(rc, "pkv_alloc_create")
        self.num_pages = num_pages
        self.page_size = page_size

    def close(self):
        if self._h:
            lib().pkv_alloc_destroy(self._h)
            self._h = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reserve(self, seq, n_tokens, max_pages=None):
        """Grow ``seq`` to ``n_tokens`` tokens; returns its table (list of page ids)."""
        width = max_pages if max_pages is not None else max(1, -(-n_tokens // self.page_size) + 1)
        row = np.full(width, -1, np.int32)
        n = ctypes.c_int32(0)
        _check(lib().pkv_alloc_reserve(self._h, seq, n_tokens, row.ctypes.data_as(_ip), width, ctypes.byref(n)),
               "pkv_alloc_reserve")
        if max_pages is None:
            return self.table(seq)
        return row[:n.value].tolist()

    def reserve_batch(self, seqs, n_tokens, block_table):
        """All-or-nothing reservation for a batch; fills ``block_table`` [B][max_pages] (int32 numpy)."""
        s, sp = _host_i32(seqs, "seqs")
        t, tp = _host_i32(n_tokens, "n_tokens")
        if block_table.dtype != np.int32 or not block_table.flags.c_contiguous:
            raise ValueError("block_table must be a C-contiguous int32 array")
        _check(lib().pkv_alloc_reserve_batch(self._h, len(s), sp, tp, block_table.ctypes.data_as(_ip),
                                             block_table.shape[1]), "pkv_alloc_reserve_batch")
        return block_table

    def share_prefix(self, seq, pages):
        arr, ptr = _host_i32(pages, "pages")
        _check(lib().pkv_alloc_share_prefix(self._h, seq, ptr, len(arr)), "pkv_alloc_share_prefix")

    def free(self, seq):
        _check(lib().pkv_alloc_free(self._h, seq), "pkv_alloc_free")

    def free_count(self):
        return int(lib().pkv_alloc_free_count(self._h))

    def table(self, seq):
        n = ctypes.c_int32(0)
        _check(lib().pkv_alloc_table(self._h, seq, None, 0, ctypes.byref(n)), "pkv_alloc_table")
        row = np.full(max(1, n.value), -1, np.int32)
        _check(lib().pkv_alloc_table(self._h, seq, row.ctypes.data_as(_ip), len(row), ctypes.byref(n)),
               "pkv_alloc_table")
        return row[:n.value].tolist()

    def cache_insert(self, key, seq, n_tokens):
        _check(lib().pkv_alloc_cache_insert(self._h, int(key), seq, n_tokens), "pkv_alloc_cache_insert")

    def cache_lookup(self, key):
        """(pages, n_tokens) kept under ``key``, or None."""
        n = ctypes.c_int32(0)
        t = ctypes.c_int32(0)
        rc = lib().pkv_alloc_cache_lookup(self._h, int(key), None, 0, ctypes.byref(n), ctypes.byref(t))
        if rc == PKV_ERR_NOT_FOUND:
            return None
        _check(rc, "pkv_alloc_cache_lookup")
        pages = np.zeros(max(1, n.value), np.int32)
        _check(lib().pkv_alloc_cache_lookup(self._h, int(key), pages.ctypes.data_as(_ip), len(pages),
                                            ctypes.byref(n), ctypes.byref(t)), "pkv_alloc_cache_lookup")
        return pages[:n.value].tolist(), t.value

    def cache_evict(self, key):
        _check(lib().pkv_alloc_cache_evict(self._h, int(key)), "pkv_alloc_cache_evict")

    def cache_entries(self):
        return int(lib().pkv_alloc_cache_entries(self._h))

    def prepare_append(self, seqs, pos, block_table=None):
        """Copy on write for a batch about to write token pos[i] of seqs[i]; returns the
        (src, dst) page copies to perform, and rewrites the batch rows of ``block_table``."""
        s, sp = _host_i32(seqs, "seqs")
        t, tp = _host_i32(pos, "pos")
        if s.shape != t.shape:
            raise ValueError("seqs and pos must have one length")
        src = np.zeros(max(1, len(s)), np.int32)
        dst = np.zeros(max(1, len(s)), np.int32)
        n = ctypes.c_int32(0)
        if block_table is not None:
            if block_table.dtype != np.int32 or not block_table.flags.c_contiguous:
                raise ValueError("block_table must be a C-contiguous int32 array")
            bp, width = block_table.ctypes.data_as(_ip), block_table.shape[1]
        else:
            bp, width = None, 0
        _check(lib().pkv_alloc_prepare_append(self._h, len(s), sp, tp, src.ctypes.data_as(_ip),
                                              dst.ctypes.data_as(_ip), ctypes.byref(n), bp, width),
               "pkv_alloc_prepare_append")
        return list(zip(src[:n.value].tolist(), dst[:n.value].tolist()))

    def refcount(self, page):
        c = ctypes.c_int32(0)
        _check(lib().pkv_alloc_refcount(self._h, page, ctypes.byref(c)), "pkv_alloc_refcount")
        return c.value


def validate_tables(block_table, lens, page_size, num_pages, exclusive_tail=False, prefix_tokens=0, window=0):
    """pkv_validate_tables on host copies; returns ``(status, row, entry, rule)``."""
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    ln, lp = _host_i32(lens, "lens")
    row, entry, rule = ctypes.c_int32(-1), ctypes.c_int32(-1), ctypes.c_int32(0)
    rc = lib().pkv_validate_tables(bt.ctypes.data_as(_ip), lp, bt.shape[0], bt.shape[1], page_size, num_pages,
                                   1 if exclusive_tail else 0, int(prefix_tokens), int(window), ctypes.byref(row),
                                   ctypes.byref(entry), ctypes.byref(rule))
    return rc, row.value, entry.value, rule.value
