"""csa2_sparse_decode_noalloc (the decode on the library's fixed per-device
scratch, for callers that cannot allocate) against csa2_sparse_decode with
a workspace: the same kernels under the same plan, so outputs and LSE agree
bit for bit.  Two calls in a row on the one scratch, the second on a smaller
input, under plans that split every sequence, so that the partials do go
through the scratch."""
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen

from gpu_common import DEV, GpuCache, decode_plan, log, to_dev

pytestmark = pytest.mark.gpu

# (B, L, K): the first call, then a smaller one (fewer sequences, shorter
# contexts, smaller K), both at H = 64, D = 512
CALLS = [(24, 6000, 1024), (5, 2500, 256)]


def _inputs(B, L, K):
    wl = gen.WORKLOADS["b8_64k"].with_(B=B, L=L, L_min=max(1, L // 3), ragged=True)
    gc = GpuCache(wl, keep_kv=False)
    ws = csa2.Workspace(DEV)
    idx, cnt = csa2.index_topk(gc.cache, gc.ctx, int(gc.lens.max()), to_dev(gen.idx_query(wl)),
                               K, ws)
    return gc, to_dev(gen.query(wl)), float(gen.softmax_scale(wl)), idx, cnt


@pytest.mark.parametrize("plan", ["auto", "hg64_split3", "hg64_split1", "hg16_split2", "hg64"])
def test_noalloc_matches_workspace_entry(plan):
    cases = [_inputs(*c) for c in CALLS]
    want, got = [], []
    with decode_plan(plan):
        for (B, L, K), (gc, q, sigma, idx, cnt) in zip(CALLS, cases):
            need = csa2.lib().csa2_sparse_decode_workspace_size(B, 64, 512, K)
            log(f"noalloc plan={plan} B={B} L={L} K={K}: partials {need} B")
            assert 0 < need <= csa2.NOALLOC_SCRATCH_BYTES
            assert need > 256              # a split plan: the partials use the scratch
            want.append(csa2.sparse_decode(gc.cache, gc.ctx, q, sigma, idx, cnt, gc.swa[0],
                                           csa2.Workspace(DEV)))
        torch.cuda.synchronize()
        # both allocation-free calls back to back on one stream, outputs made first
        outs = [(torch.full((B, 64, 512), float("nan"), device=DEV),
                 torch.full((B, 64), float("nan"), device=DEV)) for (B, _, _) in CALLS]
        for (gc, q, sigma, idx, cnt), (o, l) in zip(cases, outs):
            got.append(csa2.sparse_decode_noalloc(gc.cache, gc.ctx, q, sigma, idx, cnt,
                                                  gc.swa[0], o, l))
        torch.cuda.synchronize()
    for n, ((wo, wl), (go, gl)) in enumerate(zip(want, got)):
        assert torch.isfinite(wo).all() and torch.isfinite(wl).all()
        assert torch.equal(go, wo), f"call {n}: out differs"
        assert torch.equal(gl, wl), f"call {n}: lse differs"


def test_noalloc_without_lse_and_oversize_rejected():
    gc, q, sigma, idx, cnt = _inputs(*CALLS[1])
    B, _, K = CALLS[1]
    with decode_plan("hg64_split3"):
        wo, _ = csa2.sparse_decode(gc.cache, gc.ctx, q, sigma, idx, cnt, gc.swa[0],
                                   csa2.Workspace(DEV), want_lse=False)
        o = torch.empty((B, 64, 512), device=DEV)
        csa2.sparse_decode_noalloc(gc.cache, gc.ctx, q, sigma, idx, cnt, gc.swa[0], o, None)
        torch.cuda.synchronize()
        assert torch.equal(o, wo)
        # one-tile runs over 2K selected rows for 24 sequences need more
        # partials than the scratch holds: refused before anything runs
        gc2, q2, s2, idx2, cnt2 = _inputs(24, 6000, 2048)
    with decode_plan("hg64_split1"):
        assert csa2.lib().csa2_sparse_decode_workspace_size(24, 64, 512, 2048) > \
            csa2.NOALLOC_SCRATCH_BYTES
        with pytest.raises(csa2.Csa2Error, match="SCRATCH"):
            csa2.sparse_decode_noalloc(gc2.cache, gc2.ctx, q2, s2, idx2, cnt2, gc2.swa[0],
                                       torch.empty((24, 64, 512), device=DEV), None)
