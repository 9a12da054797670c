"""Paged-KV decode attention for AMD MI355X (gfx950).

The computation lives in the C-ABI library ``libpagedkv.so`` (hand-written
HIP kernels plus a host block allocator, declared in ``include/pagedkv.h``);
this package is its thin Python binding. Functions raise if the library has
not been built (``python -m paged_kv_cache_17_amd.build``).
"""
from .binding import (  # noqa: F401
    EXPORTED,
    KVPool,
    PKV_BF16,
    PKV_F32,
    PagedKVError,
    kv_append,
    kv_append_q8,
    kv_copy_blocks,
    kv_copy_blocks_q8,
    load_library,
    paged_attn_chunk,
    paged_attn_chunk_append,
    paged_attn_chunk_q8,
    paged_attn_chunk_q8_append,
    paged_attn_chunk_q8_workspace_size,
    paged_attn_chunk_workspace_size,
    paged_attn_decode,
    paged_attn_decode_append, paged_attn_decode_q8_append, paged_attn_decode_q8, paged_attn_decode_append_noalloc,
    paged_attn_split_tokens,
    paged_attn_workspace_size,
    pkv_set_profile_events,
    pkv_stream_read,
    sample_tokens,
    sample_workspace_size,
    strerror,
)
from .cache import PagedKVCache  # noqa: F401
