"""GPU parity at the limits of csa2_index_topk: a context of 2^24 positions
(the largest the library accepts) with the largest K (65536), checked in
full against the oracle; and the decode at its widest head count with
D = 512."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen
from oracle import select as OS

from gpu_common import DEV, GpuCache, log, to_dev, to_host

pytestmark = pytest.mark.gpu

MAX_CTX = 1 << 24
MAX_K = 65536


def test_max_context_max_k():
    """Only the indexer keys matter here: the latent rows are appended as
    zeros (the selection never reads them)."""
    wl = gen.WORKLOADS["tiny"].with_(B=1, L=MAX_CTX, D=128, Di=64, K=MAX_K)
    log(f"limits: building a {MAX_CTX}-position cache")
    pt, npages = gen.page_table(wl)
    cache = csa2.Cache.allocate(1, pt.shape[1], npages, wl.D, wl.Di, torch.from_numpy(pt), DEV)
    keys = gen.idx_keys(wl, 0, MAX_CTX)
    step = 1 << 22
    zeros = torch.zeros((step, wl.D), dtype=torch.uint16, device=DEV)
    seq = torch.zeros(step, dtype=torch.int32, device=DEV)
    for i in range(0, MAX_CTX, step):
        csa2.quantize_append(cache, zeros, seq,
                             torch.arange(i, i + step, dtype=torch.int32, device=DEV),
                             keys=to_dev(keys[i:i + step]))
    ctx = torch.full((1,), MAX_CTX, dtype=torch.int32, device=DEV)
    q = gen.idx_query(wl)
    log("limits: index_topk at max_ctx, K = 65536")
    idx, cnt = csa2.index_topk(cache, ctx, MAX_CTX, to_dev(q), MAX_K, csa2.Workspace(DEV))
    torch.cuda.synchronize()
    n = MAX_CTX - gen.WINDOW
    sc = np.concatenate([OS.indexer_scores(q[0], keys[i:min(n, i + step)])
                         for i in range(0, n, step)])
    want, wcnt = OS.topk(sc, MAX_CTX, MAX_K)
    assert int(to_host(cnt)[0]) == wcnt == MAX_K
    assert np.array_equal(to_host(idx)[0], want)


def test_decode_widest_heads_d512():
    from test_gpu_decode import _decode_and_check
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=3000, D=512, H=128, Di=128)
    log("limits: decode D=512 H=128")
    _decode_and_check(GpuCache(wl), 1024)
