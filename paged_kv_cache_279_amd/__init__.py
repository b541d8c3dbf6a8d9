"""Paged KV-cache single-token decode attention for AMD MI355X (gfx950).

The kernels and the page allocator live in ``libpkv.so`` (C ABI, ``include/pkv.h``);
this package is its Python binding. Build it with
``python -m paged_kv_cache_279_amd.build``.
"""

from .binding import (  # noqa: F401
    PKV_OK,
    PKV_ERR_INVALID_ARG,
    PKV_ERR_UNSUPPORTED,
    PKV_ERR_OUT_OF_PAGES,
    PKV_ERR_WORKSPACE_TOO_SMALL,
    PKV_ERR_HIP,
    PKV_ERR_INVALID_TABLE,
    PKV_ERR_NOT_FOUND,
    PKV_ERR_HOST_MEMORY,
    PKV_ERR_SCRATCH_LIMIT,
    PkvError,
    PageAllocator,
    append_paged_decode_attention,
    block_table_patch,
    copy_pages,
    decode_workspace_bytes,
    decode_workspace_bytes_multi,
    empty_pool,
    k8_pool_bytes,
    kv_append,
    kv_append_chunk,
    kv_append_k8,
    kv_append_k8_chunk,
    lib,
    paged_decode_attention,
    paged_decode_attention_k8,
    paged_decode_attention_multi,
    paged_decode_attention_multi_k8,
    paged_decode_attention_shared_prefix,
    paged_decode_attention_shared_prefix_noalloc,
    noalloc_scratch_bytes,
    paged_decode_attention_window,
    paged_decode_attention_window_multi,
    paged_decode_attention_window_k8,
    pool_shape,
    probe_stream_read,
    profile_next_partition_kernel,
    status_string,
    validate_tables,
)
