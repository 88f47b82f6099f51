"""pkv — paged-KV decode attention for AMD MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (``include/pkv.h``, ``libpkv.so``); this package is the
thin Python binding with the same entry-point names.  Importing it fails if the library has not
been built (``python paged_kv_cache_203_amd/build.py``): there is no fallback implementation.
"""
from ._lib import (LIB_PATH, PkvError, PkvShape, STATUS_APPEND_ALIAS, STATUS_CAPACITY,  # noqa: F401
                   STATUS_PAGE_RANGE, last_error, lib, lse_merge, make_shape,
                   paged_decode_attention, paged_decode_attention_partial, paged_decode_cascade,
                   paged_decode_multi_query, paged_decode_multi_query_step,
                   multi_query_step_workspace_bytes,
                   paged_decode_step, paged_decode_step_noalloc,
                   decode_step_workspace_bytes,
                   paged_decode_attention_split, paged_kv_append, partial_workspace_bytes,
                   rope_kv_append, copy_pages, PageAllocator, read_stream,
                   partitions_needed, validate_metadata, version)
