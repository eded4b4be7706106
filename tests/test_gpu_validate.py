"""GPU check of csa2_validate_selection: a selection made by csa2_index_topk
passes; each planted contract violation (inputs that the other kernels
survive by skipping them) sets exactly its bit on its sequence only."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from fp4_compressed_sparse_csa2_amd import _lib
from harness import gen

from gpu_common import DEV, GpuCache, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_planted_violations():
    wl = gen.WORKLOADS["b128_rag"].with_(B=8, L=9000, L_min=3000, D=128, H=16, Di=64)
    log("validate selection")
    gc = GpuCache(wl, keep_kv=False)
    K = 512
    idx, cnt = csa2.index_topk(gc.cache, gc.ctx, int(gc.lens.max()), to_dev(gen.idx_query(wl)),
                               K, csa2.Workspace(DEV))
    assert not to_host(csa2.validate_selection(gc.cache, gc.ctx, idx, cnt)).any()

    idx_h, cnt_h, lens = to_host(idx).copy(), to_host(cnt).copy(), gc.lens.astype(np.int32).copy()
    want = np.zeros(wl.B, np.int64)
    cnt_h[0] = K + 1;                               want[0] = _lib.SEL_BAD_COUNT
    idx_h[1, cnt_h[1] - 1] = int(lens[1]) - 5;      want[1] = _lib.SEL_BAD_POSITION  # in the window
    idx_h[2, 0] = -4;                               want[2] = _lib.SEL_BAD_POSITION
    idx_h[3, [10, 11]] = idx_h[3, [11, 10]];        want[3] = _lib.SEL_NOT_ASCENDING
    idx_h[4, 20] = idx_h[4, 19];                    want[4] = _lib.SEL_NOT_ASCENDING  # a duplicate
    lens[5] = -1;                                   want[5] = _lib.SEL_BAD_LENGTH | _lib.SEL_BAD_POSITION
    flags = to_host(csa2.validate_selection(gc.cache, to_dev(lens), to_dev(idx_h), to_dev(cnt_h)))
    assert np.array_equal(flags, want), (flags, want)

    # a shard's view of the cache: pages it does not hold are -1
    pt = gc.pt.copy()
    pt[6, : pt.shape[1] // 2] = -1
    view = csa2.Cache(gc.cache.pages, to_dev(pt), wl.D, wl.Di)
    flags = to_host(csa2.validate_selection(view, gc.ctx, idx, cnt))
    assert flags[6] == _lib.SEL_BAD_PAGE and not np.delete(flags, 6).any()


def test_window_ring_range():
    """csa2_validate_window flags a live window value that fp16 does not hold
    exactly (above 65504, or too fine below 2^-14) and non-finite values, not
    dead slots; rings at the edge of the range (65280, 2^-24, 2^-14 - 2^-24
    steps) pass and decode within the bar against the oracle."""
    from gpu_common import ATOL, assert_close, oracle_decode, oracle_topk
    wl = gen.WORKLOADS["tiny"].with_(B=6, L=1000)
    log("validate window ring range")
    gc = GpuCache(wl)
    lens = gc.lens.astype(np.int32).copy()
    lens[5] = 50                                      # slots >= 50 are dead
    # the N(0,1) draw holds a few values below 2^-14 that fp16 subnormals do
    # not hold exactly (about one per 16K): zero them, so that only the
    # planted values decide the flags
    base = gc.rings[0].copy()
    base[np.abs(gen.bf16_bits_to_f32(base)) < 2.0 ** -14] = 0
    ring = base.copy()
    bf = lambda v: gen.f32_to_bf16_bits(np.array([v], np.float32))[0]
    edge = [bf(65280.0), bf(-65280.0), bf(2.0 ** -24), bf(-(2.0 ** -14)), bf(3 * 2.0 ** -24)]
    ring[0, 7, :len(edge)] = edge                     # exact in fp16: no flag
    ring[1, 3, 5] = bf(70000.0)                       # above 65504
    ring[2, 100, 9] = bf(1e-6)                        # below 2^-14, not a multiple of 2^-24
    ring[3, 0, 0] = 0x7F80                            # +inf
    ring[4, 1, 1] = 0x7FC1                            # NaN
    ring[5, 60, 0] = 0x7FC1                           # a dead slot: not read
    flags = to_host(csa2.validate_window(gc.cache, to_dev(lens), to_dev(ring)))
    want = np.array([0, _lib.WIN_NOT_F16, _lib.WIN_NOT_F16, _lib.WIN_NOT_FINITE,
                     _lib.WIN_NOT_FINITE, 0])
    assert np.array_equal(flags, want), flags

    # the edge values decode within the bar, taken relative to the output's
    # magnitude here: the f16 weights that multiply the rows carry a relative
    # rounding of 2^-12, so a row of magnitude 65280 moves an output by up to
    # 16 times its weight, against about 1e-3 for the N(0,1) rows the absolute
    # 2e-3 is set for.  The query is scaled by 2^-12 so that the value 65280
    # does not take the whole softmax (outputs stay near 200).
    edge_ring = base.copy()
    edge_ring[:, 7, :len(edge)] = edge
    q = gen.f32_to_bf16_bits(gen.bf16_bits_to_f32(gen.query(wl)) * np.float32(2.0 ** -12))
    qi = gen.idx_query(wl)
    sigma = float(gen.softmax_scale(wl))
    idx, cnt = csa2.index_topk(gc.cache, gc.ctx, int(gc.lens.max()), to_dev(qi), wl.K,
                               csa2.Workspace(DEV))
    out, lse = csa2.sparse_decode(gc.cache, gc.ctx, to_dev(q), sigma, idx, cnt, to_dev(edge_ring),
                                  csa2.Workspace(DEV))
    assert not to_host(csa2.validate_window(gc.cache, gc.ctx, to_dev(edge_ring))).any()
    idx_h, cnt_h, out_h, lse_h = map(to_host, (idx, cnt, out, lse))
    for b in range(wl.B):
        L = int(gc.lens[b])
        _, want, wcnt = oracle_topk(gc.keys[b], qi[b], L, wl.K)
        assert int(cnt_h[b]) == wcnt and np.array_equal(idx_h[b], want)
        sel = want[:wcnt]
        o, l = oracle_decode(q[b], sigma, gc.kv_rows(b, sel), edge_ring[b], sel, L)
        assert_close(out_h[b], o, ATOL * max(1.0, float(np.max(np.abs(o)))),
                     f"edge ring out b={b}")
        assert_close(lse_h[b], l, ATOL, f"edge ring lse b={b}")
