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
