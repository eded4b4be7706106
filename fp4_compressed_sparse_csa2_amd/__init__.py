"""CSA2 sparse decode over an FP4 E2M1 / E4M3-per-16 global KV cache, native
to AMD MI355X (gfx950).

The compute path is the HIP library ``libcsa2.so`` (C ABI in
``include/csa2.h``); this package is its Python binding.  Importing it does
not load the library; the first call does, and fails loudly if it is missing.
"""
from ._lib import (  # noqa: F401
    PAGE_TOKENS,
    WINDOW,
    Cache,
    Csa2Error,
    Workspace,
    append_index_topk,
    index_topk,
    index_topk_range,
    index_topk_range_scaled,
    index_topk_scaled,
    key_scales_for,
    lib,
    lse_merge,
    page_bytes,
    quantize_append,
    reindex,
    reindex_scaled,
    restore_window,
    NOALLOC_SCRATCH_BYTES,
    sparse_decode,
    sparse_decode_noalloc,
    store_key_scales,
    stream_read,
    topk_merge,
    validate_selection,
    validate_window,
    workspace_init,
)
