"""The library's calls captured in a HIP graph: every replay (with eager
work and synchronisations in between) reproduces the eager results bit for
bit, so the workspaces' control words are returned to zero inside the
captured kernels and no call depends on host-side state."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen

from gpu_common import DEV, GpuCache, log, to_dev

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    wl = gen.WORKLOADS["b128_rag"].with_(B=6, L=40000, L_min=20000, D=512, H=64, Di=128)
    log("graph replays of a decode step")
    gc = GpuCache(wl, keep_kv=False)
    B, K, max_ctx = wl.B, wl.K, int(gc.lens.max())
    x, k = gen.append_tokens(wl, 0)
    seq = torch.arange(B, dtype=torch.int32, device=DEV)
    pos = to_dev((gc.lens - 1).astype(np.int32))           # rewrite the last token
    xd, kd = to_dev(x), to_dev(k)
    q_idx, q = to_dev(gen.idx_query(wl)), to_dev(gen.query(wl))
    q1 = to_dev(gen.idx_query(wl, 1))
    sigma = float(gen.softmax_scale(wl))
    ks = csa2.key_scales_for(gc.cache)
    ks.fill_(0.5)
    idx = torch.empty((B, K), dtype=torch.int32, device=DEV)
    cnt = torch.empty((B,), dtype=torch.int32, device=DEV)
    idx2 = torch.empty((B, 256), dtype=torch.int32, device=DEV)
    cnt2 = torch.empty((B,), dtype=torch.int32, device=DEV)
    sidx = torch.empty((B, K), dtype=torch.int32, device=DEV)
    scnt = torch.empty((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, wl.H, wl.D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, wl.H), dtype=torch.float32, device=DEV)
    ws = [csa2.Workspace(DEV) for _ in range(4)]

    def step():
        csa2.append_index_topk(gc.cache, xd, seq, pos, kd, gc.swa[0], gc.ctx, max_ctx, q_idx, K,
                               ws[0], out_idx=idx, out_count=cnt)
        csa2.reindex(gc.cache, q1, idx, cnt, 256, ws[1], out_idx=idx2, out_count=cnt2)
        csa2.index_topk_scaled(gc.cache, gc.ctx, max_ctx, q1, ks, K, ws[2], out_idx=sidx,
                               out_count=scnt)
        csa2.sparse_decode(gc.cache, gc.ctx, q, sigma, idx, cnt, gc.swa[0], ws[3], out=out, lse=lse)

    step()                                                 # eager (sizes the workspaces)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (idx, cnt, idx2, cnt2, sidx, scnt, out, lse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (idx, cnt, idx2, cnt2, sidx, scnt, out, lse):
            t.zero_()                                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (idx, cnt, idx2, cnt2, sidx, scnt, out, lse)
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {rep} differs"
        step()                                             # eager again on the same workspaces
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"eager after replay {rep}"
