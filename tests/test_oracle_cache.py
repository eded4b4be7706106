"""Pins for the oracle's cache writes: an appended row equals a bulk
quantisation of the same token, window slots hold the input bits, and keys
land next to their rows."""
import numpy as np

from harness import gen
from oracle import cache as C
from oracle import formats as F


def test_append_roundtrip_paged():
    wl = gen.WORKLOADS["tiny"].with_(L=300, paged=True, append_steps=0)
    lens = gen.ctx_lens(wl)
    pt, npages = gen.page_table(wl, lens)
    D, Di = wl.D, wl.Di
    pages = np.zeros((npages, C.page_bytes(D, Di)), np.uint8)
    swa = np.zeros((1, 128, D), np.uint16)
    kv = gen.kv_bf16(wl, 0, 300)
    keys = gen.idx_keys(wl, 0, 300)
    pos = np.arange(300)
    C.append(pages, pt, D, Di, np.zeros(300, int), pos, kv, keys, swa)
    codes, scales = C.rows_of(pages, pt, D, Di, 0, pos)
    c2, s2 = F.quantize_rows(kv)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    assert np.array_equal(C.keys_of(pages, pt, D, Di, 0, pos), keys)
    assert np.array_equal(swa[0], gen.swa_ring(wl, kv, 300))
    assert C.page_bytes(512, 128) == 26624 and C.page_bytes(128, 64) == 8704


def test_row_byte_index_matches_rows_of():
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=700, paged=True, append_steps=0)
    lens = gen.ctx_lens(wl)
    pt, npages = gen.page_table(wl, lens)
    D, Di = wl.D, wl.Di
    pages = np.random.default_rng(3).integers(0, 256, (npages, C.page_bytes(D, Di))).astype(np.uint8)
    pos = np.array([0, 1, 63, 64, 65, 300, 699])
    for b in range(2):
        ci, si = C.row_byte_index(pt, D, Di, b, pos)
        codes, scales = C.rows_of(pages, pt, D, Di, b, pos)
        flat = pages.reshape(-1)
        assert np.array_equal(flat[ci], codes) and np.array_equal(flat[si], scales)
