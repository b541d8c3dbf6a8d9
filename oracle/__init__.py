"""CPU fp64 oracle for paged-KV single-token decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
anything in this package. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the HIP
path (``paged_kv_cache_279_amd``): it imports neither that package nor torch,
and works on plain numpy arrays in float64.

Sources (the three web pages on LLM-inference optimisation this build follows):
  hotelren  = www.hotelren.com/news/4669576  (site title 企业官网建设流程全解析)
  dpshk     = www.dpshk.com/news/5622214     (same site title)
  pgsm      = www.pgsm.cn/news/396587
              "LLM推理优化：从硬件瓶颈到KV Cache的工程实践"
Citations below name the page key and the section number on that page.

Every function here is pinned by ``tests/test_oracle_*.py`` to something other
than itself (closed forms the pages print, brute force on tiny inputs,
invariances, textbook special cases, a library attention routine). No function
is "parity unpinned".
"""

from .paged_decode import (  # noqa: F401
    kv_cache_bytes,
    pages_for_tokens,
    pool_bytes,
    pool_dims,
    pool_shape,
    token_slot,
    k_tile_offset,
    v_tile_offset,
    read_token,
    write_token,
    gather_sequence,
    decode_attention,
    decode_attention_multi,
    decode_attention_window,
    decode_attention_window_multi,
    kv_append,
    decode_partials,
    lse_merge,
)
from .quant_k8 import (  # noqa: F401
    k8_subblock_bytes,
    k8_pool_bytes,
    k8_code_offset,
    k8_scale_offset,
    quantize_k,
    k8_write_token,
    k8_read_token,
    quantize_k_pool,
    k8_gather_sequence,
    decode_attention_k8,
    decode_attention_multi_k8,
    decode_attention_window_k8,
    decode_attention_window_multi_k8,
    kv_append_k8,
)
from .allocator import PageAllocatorModel, OutOfPages, validate_tables  # noqa: F401
