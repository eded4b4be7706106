"""The C-ABI library without a GPU: it loads, exports every entry point that
include/csa2.h declares, and its host-side validation rejects bad arguments
before anything is launched (these calls reach no HIP API)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import fp4_compressed_sparse_csa2_amd as csa2
    if not os.path.exists(csa2._lib.LIB_PATH):
        pytest.skip("libcsa2.so not built")
    return csa2.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) == 25, names
    for n in names:
        assert hasattr(L, n), n


def test_page_bytes_and_strings(L):
    assert L.csa2_page_bytes(512, 128) == 64 * (256 + 32 + 128)
    assert L.csa2_page_bytes(128, 64) == 64 * (64 + 8 + 64)
    assert L.csa2_page_bytes(100, 64) == 0 and L.csa2_page_bytes(512, 96) == 0
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert L.csa2_status_string(s).startswith(b"CSA2_")


def test_workspace_sizes(L):
    assert L.csa2_index_topk_workspace_size(8, 65536, 2048) > 8 * 65536 * 12
    assert L.csa2_index_topk_workspace_size(0, 100, 1) == 0
    assert L.csa2_reindex_workspace_size(8, 8192, 2048) >= 8 * 8192 * 4
    assert L.csa2_reindex_workspace_size(8, 100, 200) == 0          # K > P
    assert L.csa2_sparse_decode_workspace_size(8, 64, 512, 2048) > 0
    assert L.csa2_sparse_decode_workspace_size(8, 24, 512, 2048) == 0   # H not a multiple of 16
    assert L.csa2_sparse_decode_workspace_size(8, 64, 384, 2048) == 0   # unsupported D


def _cache(D=512, Di=128, batch=1, pages=1, table=1):
    from fp4_compressed_sparse_csa2_amd._lib import CacheStruct
    return CacheStruct(pages, table, 4, 4, batch, D, Di)


def test_validation_codes(L):
    c = _cache()
    P = ctypes.byref
    assert L.csa2_quantize_append(None, 1, 1, None, 1, 1, None, None) == -1
    assert L.csa2_quantize_append(P(_cache(pages=0)), 1, 1, None, 1, 1, None, None) == -1
    assert L.csa2_quantize_append(P(_cache(D=384)), 1, 1, None, 1, 1, None, None) == -3
    assert L.csa2_quantize_append(P(_cache(batch=0)), 1, 1, None, 1, 1, None, None) == -2
    assert L.csa2_quantize_append(P(c), -1, 1, None, 1, 1, None, None) == -2
    assert L.csa2_quantize_append(P(c), 1, None, None, 1, 1, None, None) == -1
    # index_topk: K out of range, workspace missing / too small
    assert L.csa2_index_topk(P(c), 1, 100, 1, -1, 1, 1, None, 1, 1 << 30, None) == -2
    assert L.csa2_index_topk(P(c), 1, 100, 1, 8, 1, 1, None, None, 0, None) == -4
    assert L.csa2_index_topk(P(c), 1, 100, 1, 8, 1, 1, None, 1, 16, None) == -4
    # reindex: K > P
    assert L.csa2_reindex(P(c), 1, 1, 1, 10, 20, 1, 1, None, 1, 1 << 30, None) == -2
    # sparse_decode: H not a multiple of 16, null output
    assert L.csa2_sparse_decode(P(c), 1, 24, 1, 1.0, 1, 1, 8, 1, 1, None, 1, 1 << 30, None) == -3
    assert L.csa2_sparse_decode(P(c), 1, 16, 1, 1.0, 1, 1, 8, 1, None, None, 1, 1 << 30, None) == -1


def test_shard_calls_validate_before_launch(L):
    c = _cache()
    P = ctypes.pointer
    # index_topk_range: p_begin not page-aligned, p_end below p_begin, null output
    assert L.csa2_index_topk_range(P(c), 1, 100, 1, 8, 32, 200, 1, 1, None, 1, 1 << 30, None) == -2
    assert L.csa2_index_topk_range(P(c), 1, 100, 1, 8, 64, 10, 1, 1, None, 1, 1 << 30, None) == -2
    assert L.csa2_index_topk_range(P(c), 1, 100, 1, 8, 0, 10, None, 1, None, 1, 1 << 30, None) == -1
    # topk_merge: sizes and workspace
    assert L.csa2_topk_merge_workspace_size(8, 4, 2048, 2048) > 0
    assert L.csa2_topk_merge_workspace_size(8, 0, 2048, 2048) == 0
    assert L.csa2_topk_merge_workspace_size(8, 65, 16, 16) == 0
    assert L.csa2_topk_merge_workspace_size(8, 2, 16, 40) == 0          # K > n * K_in
    assert L.csa2_topk_merge(8, 2, 16, 1, 1, 1, 40, 1, 1, None, 1, 1 << 30, None) == -2
    assert L.csa2_topk_merge(8, 2, 16, 1, 1, None, 8, 1, 1, None, 1, 1 << 30, None) == -1
    assert L.csa2_topk_merge(8, 2, 16, 1, 1, 1, 8, 1, 1, None, None, 0, None) == -4
    # lse_merge: null input, unsupported D, part count
    assert L.csa2_lse_merge(2, 8, 64, 512, None, 1, 1, None, None) == -1
    assert L.csa2_lse_merge(2, 8, 64, 384, 1, 1, 1, None, None) == -3
    assert L.csa2_lse_merge(0, 8, 64, 512, 1, 1, 1, None, None) == -2



def test_scaled_calls_validate_before_launch(L):
    c = _cache()
    P = ctypes.pointer
    # store_key_scales: negative count, null input
    assert L.csa2_store_key_scales(P(c), -1, 1, 1, 1, 1, None) == -2
    assert L.csa2_store_key_scales(P(c), 4, 1, 1, 1, None, None) == -1
    assert L.csa2_store_key_scales(P(c), 0, None, None, None, None, None) == 0   # nothing to do
    assert L.csa2_store_key_scales_e4m3(P(c), -1, 1, 1, 1, 1, None) == -2
    assert L.csa2_store_key_scales_e4m3(P(c), 4, None, 1, 1, 1, None) == -1
    # index_topk_scaled: null scales, K out of range, short workspace
    assert L.csa2_index_topk_scaled(P(c), 1, 100, 1, None, 8, 1, 1, None, None, 1, 1 << 30,
                                    None) == -1
    assert L.csa2_index_topk_scaled(P(c), 1, 100, 1, 1, -1, 1, 1, None, None, 1, 1 << 30,
                                    None) == -2
    assert L.csa2_index_topk_scaled(P(c), 1, 100, 1, 1, 8, 1, 1, None, None, 1, 16, None) == -4
    # reindex_scaled: null scales, K > P
    assert L.csa2_reindex_scaled(P(c), 1, None, 1, 1, 10, 8, 1, 1, None, 1, 1 << 30, None) == -1
    assert L.csa2_reindex_scaled(P(c), 1, 1, 1, 1, 10, 20, 1, 1, None, 1, 1 << 30, None) == -2


def test_append_index_topk_validates_before_launch(L):
    c = _cache()
    P = ctypes.pointer
    # negative token count, null token input, K out of range, short workspace
    assert L.csa2_append_index_topk(P(c), -1, 1, None, 1, 1, None, 1, 100, 1, 8, 1, 1, None, 1,
                                    1 << 30, None) == -2
    assert L.csa2_append_index_topk(P(c), 4, None, None, 1, 1, None, 1, 100, 1, 8, 1, 1, None, 1,
                                    1 << 30, None) == -1
    assert L.csa2_append_index_topk(P(c), 4, 1, None, 1, 1, None, 1, 100, 1, -1, 1, 1, None, 1,
                                    1 << 30, None) == -2
    assert L.csa2_append_index_topk(P(c), 4, 1, None, 1, 1, None, 1, 100, 1, 8, 1, 1, None, 1,
                                    16, None) == -4


def test_sharded_scaled_calls_validate_before_launch(L):
    c = _cache()
    P = ctypes.pointer
    # range: null scales, p_begin not page-aligned; merge of values: K > n * K_in
    assert L.csa2_index_topk_range_scaled(P(c), 1, 100, 1, None, 8, 0, 64, 1, 1, None, 1,
                                          1 << 30, None) == -1
    assert L.csa2_index_topk_range_scaled(P(c), 1, 100, 1, 1, 8, 32, 200, 1, 1, None, 1,
                                          1 << 30, None) == -2
    assert L.csa2_topk_merge_values(8, 2, 16, 1, 1, 1, 40, 1, 1, None, 1, 1 << 30, None) == -2
    assert L.csa2_topk_merge_values(8, 2, 16, 1, 1, None, 8, 1, 1, None, 1, 1 << 30, None) == -1


def test_stream_read_validates_before_launch(L):
    assert L.csa2_stream_read(None, 0, None, None) == 0                # nothing to read
    assert L.csa2_stream_read(None, 16, 1, None) == -1
    assert L.csa2_stream_read(16, 16, None, None) == -1
    assert L.csa2_stream_read(16, 24, 1, None) == -2                   # not a multiple of 16
    assert L.csa2_stream_read(8, 16, 1, None) == -2                    # misaligned


def test_validate_window_validates_before_launch(L):
    c = _cache()
    P = ctypes.byref
    assert L.csa2_validate_window(P(c), 1, 1, None, None) == -1          # no flags buffer
    assert L.csa2_validate_window(P(c), 1, None, 1, None) == -1          # no ring
    assert L.csa2_validate_window(P(_cache(D=384)), 1, 1, 1, None) == -3


def test_validate_selection_validates_before_launch(L):
    c = _cache()
    P = ctypes.pointer
    assert L.csa2_validate_selection(P(c), 1, 1, 1, 8, None, None) == -1      # no flags buffer
    assert L.csa2_validate_selection(P(c), 1, None, 1, 8, 1, None) == -1      # no indices
    assert L.csa2_validate_selection(P(c), 1, 1, 1, -1, 1, None) == -2


def test_noalloc_decode_validates_before_launch(L):
    """csa2_sparse_decode_noalloc checks its arguments, and that the request
    fits the fixed scratch, before it looks up or touches any device."""
    import fp4_compressed_sparse_csa2_amd as csa2
    P = ctypes.byref
    c = _cache()
    assert L.csa2_sparse_decode_noalloc(P(c), 1, 24, 1, 1.0, 1, 1, 8, 1, 1, None, None) == -3
    assert L.csa2_sparse_decode_noalloc(P(c), 1, 16, 1, 1.0, 1, 1, 8, 1, None, None, None) == -1
    assert L.csa2_sparse_decode_noalloc(P(c), 1, 16, 1, 1.0, 1, 1, -1, 1, 1, None, None) == -2
    # 128 sequences x 128 heads x D = 512 with K = 65536 takes split partials
    # far beyond the scratch
    big = _cache(batch=128)
    assert L.csa2_sparse_decode_workspace_size(128, 128, 512, 65536) > csa2.NOALLOC_SCRATCH_BYTES
    assert L.csa2_sparse_decode_noalloc(P(big), 1, 128, 1, 1.0, 1, 1, 65536, 1, 1, None,
                                        None) == -6
    assert b"SCRATCH" in L.csa2_status_string(-6)
