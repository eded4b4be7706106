"""Bounded replay: the FP4 pages and indexer keys are the persisted state; a
layer's window ring is dropped and rebuilt by re-appending the bf16 tokens of
the last 128 positions (the pages keep the window's bf16 only as FP4, so the
ring cannot be recovered from them).  Checked bit-exact: the rebuilt ring
equals the oracle's ring, the pages equal the persisted ones (re-quantising a
token writes the same bytes), and the decode on the restored state equals
the decode before the drop."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen

from gpu_common import DEV, GpuCache, log, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_short", "paged_ragged"])
def test_window_restored_by_reappending(name):
    if name == "tiny_short":
        wl = gen.WORKLOADS["tiny"].with_(B=3, L=3000)
    else:
        wl = gen.WORKLOADS["b128_rag"].with_(B=5, L=2000, L_min=40, D=128, H=16, K=256)
    log(f"bounded replay {name}")
    gc = GpuCache(wl)
    q = to_dev(gen.query(wl))
    sigma = float(gen.softmax_scale(wl))
    max_ctx = int(gc.lens.max())
    idx, cnt = csa2.index_topk(gc.cache, gc.ctx, max_ctx, to_dev(gen.idx_query(wl)), wl.K,
                               csa2.Workspace(DEV))
    out0, lse0 = csa2.sparse_decode(gc.cache, gc.ctx, q, sigma, idx, cnt, gc.swa[0],
                                    csa2.Workspace(DEV))
    torch.cuda.synchronize()
    persisted = to_host(gc.cache.pages).copy()                 # FP4 rows + keys only
    # a fresh device state from the persisted pages, the ring dropped
    cache2 = csa2.Cache(to_dev(persisted), to_dev(gc.pt), wl.D, wl.Di)
    ring2 = torch.zeros_like(gc.swa[0])
    tokens = np.zeros((wl.B, gen.WINDOW, wl.D), np.uint16)
    for b in range(wl.B):
        L = int(gc.lens[b])
        w = min(L, gen.WINDOW)
        if w:
            tokens[b, gen.WINDOW - w:] = gc.kv_rows(b, np.arange(L - w, L))
    csa2.restore_window(cache2, ring2, to_dev(tokens), gc.lens)
    out1, lse1 = csa2.sparse_decode(cache2, gc.ctx, q, sigma, idx, cnt, ring2, csa2.Workspace(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ring2), gc.rings[0]), "restored ring differs from the oracle ring"
    assert np.array_equal(to_host(cache2.pages), persisted), "re-append changed the pages"
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1), "decode after restore differs"
