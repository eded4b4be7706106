"""GPU parity of the context-sharded path against the oracle.

A sequence's candidates are cut into page-aligned, ascending position ranges
(one per emulated device).  Checked: each range's selection (positions, count
and the scores of the selected) bit-exact against the oracle's shard
selection; their merge bit-exact against the oracle's one-device Top-K and
against csa2_index_topk; attention of each shard over the merged selection
through a page-table view that holds only its own pages (the window only on
the tail shard), LSE-merged, within the decode tolerance of the fp64 oracle
over the whole selection and close to the one-device decode."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen
from oracle import select as OS

from gpu_common import ATOL, DEV, GpuCache, assert_close, log, oracle_decode, to_dev, to_host

pytestmark = pytest.mark.gpu


def _bounds(L_max: int, n: int) -> list[tuple[int, int]]:
    """n page-aligned ascending ranges; the last one is open-ended."""
    pages = -(-L_max // 64)
    cuts = [int(round(pages * i / n)) * 64 for i in range(n)]
    return [(cuts[i], cuts[i + 1] if i + 1 < n else 1 << 24) for i in range(n)]


def _run(gc: GpuCache, n: int, K: int, sample=None):
    wl = gc.wl
    B = wl.B
    max_ctx = int(gc.lens.max())
    q_idx_h, q_h = gen.idx_query(wl), gen.query(wl)
    q_idx, q = to_dev(q_idx_h), to_dev(q_h)
    sigma = float(gen.softmax_scale(wl))
    bounds = _bounds(max_ctx, n)
    parts_idx = torch.empty((n, B, K), dtype=torch.int32, device=DEV)
    parts_sc = torch.empty((n, B, K), dtype=torch.int32, device=DEV)
    parts_cnt = torch.empty((n, B), dtype=torch.int32, device=DEV)
    ws = csa2.Workspace(DEV)
    for s, (a, e) in enumerate(bounds):
        csa2.index_topk_range(gc.cache, gc.ctx, max_ctx, q_idx, K, a, e, ws, out_idx=parts_idx[s],
                              out_count=parts_cnt[s], out_sel_scores=parts_sc[s])
    midx, mcnt, msc = csa2.topk_merge(parts_idx, parts_sc, parts_cnt, K, csa2.Workspace(DEV))
    one_idx, one_cnt = csa2.index_topk(gc.cache, gc.ctx, max_ctx, q_idx, K, csa2.Workspace(DEV))
    # attention: shard s sees only the pages of [a, e); the tail shard also the window
    outs = torch.empty((n, B, wl.H, wl.D), dtype=torch.float32, device=DEV)
    lses = torch.empty((n, B, wl.H), dtype=torch.float32, device=DEV)
    for s, (a, e) in enumerate(bounds):
        pt = gc.pt.copy()
        own = np.zeros(pt.shape[1], dtype=bool)
        own[a // 64: min(pt.shape[1], -(-e // 64))] = True
        pt[:, ~own] = -1
        view = csa2.Cache(gc.cache.pages, to_dev(pt), wl.D, wl.Di)
        csa2.sparse_decode(view, gc.ctx, q, sigma, midx, mcnt, gc.swa[0] if s == n - 1 else None,
                           csa2.Workspace(DEV), out=outs[s], lse=lses[s])
    out, lse = csa2.lse_merge(outs, lses)
    one_out, one_lse = csa2.sparse_decode(gc.cache, gc.ctx, q, sigma, one_idx, one_cnt, gc.swa[0],
                                          csa2.Workspace(DEV))
    torch.cuda.synchronize()
    pi, ps, pc = to_host(parts_idx), to_host(parts_sc), to_host(parts_cnt)
    mi, mc, ms = to_host(midx), to_host(mcnt), to_host(msc)
    oi, oc = to_host(one_idx), to_host(one_cnt)
    out_h, lse_h, one_out_h, one_lse_h = map(to_host, (out, lse, one_out, one_lse))
    worst = 0.0
    for b in range(B) if sample is None else sample:
        L = int(gc.lens[b])
        sc = OS.indexer_scores(q_idx_h[b], gc.keys[b][:max(0, L - gen.WINDOW)])
        for s, (a, e) in enumerate(bounds):
            wi, wc, ws_ = OS.topk_range(sc, L, K, a, e)
            assert int(pc[s, b]) == wc, f"shard {s} count b={b}"
            assert np.array_equal(pi[s, b], wi), f"shard {s} indices b={b}"
            assert np.array_equal(ps[s, b, :wc], ws_[:wc]), f"shard {s} scores b={b}"
        want, wcnt = OS.topk(sc, L, K)
        assert int(mc[b]) == wcnt and np.array_equal(mi[b], want), f"merged Top-K b={b}"
        assert int(oc[b]) == wcnt and np.array_equal(oi[b], mi[b]), f"one-device Top-K b={b}"
        assert np.array_equal(ms[b, :wcnt], sc[want[:wcnt]]), f"merged scores b={b}"
        sel = want[:wcnt]
        o, l = oracle_decode(q_h[b], sigma, gc.kv_rows(b, sel), gc.rings[0, b], sel, L)
        worst = max(worst, assert_close(out_h[b], o, ATOL, f"merged out b={b}"))
        assert_close(lse_h[b], l, ATOL, f"merged lse b={b}")
        assert_close(out_h[b], one_out_h[b], 1e-4, f"merged vs one-device out b={b}")
    log(f"  {n} shards: selections bit-exact, merged attention max-abs error {worst:.2e}")


@pytest.mark.parametrize("n", [1, 3, 4])
def test_shards_small(n):
    wl = gen.WORKLOADS["tiny"].with_(B=3, L=9000)
    log(f"shards tiny B=3 L=9000 n={n}")
    _run(GpuCache(wl), n, 256)


def test_shards_all_equal_scores():
    """Every score equal: the merge rests on the position order alone."""
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=6000)
    log("shards with all-equal scores")
    gc = GpuCache(wl, keys_fn=lambda b, k: np.zeros_like(k))
    _run(gc, 3, 1000)


def test_shards_paged_ragged():
    """Ragged lengths on a permuted page table: some shards of the short
    sequences hold no candidates."""
    wl = gen.WORKLOADS["b128_rag"].with_(B=6, L=20000, L_min=200, D=128, H=16)
    log("shards paged ragged B=6")
    _run(GpuCache(wl), 4, 512)


def test_shards_1m_context():
    """The one-sequence, 1M-token case cut over 8 emulated devices."""
    wl = gen.WORKLOADS["b1_1m"]
    log("shards b1_1m n=8: building the cache")
    _run(GpuCache(wl, keep_kv=False), 8, wl.K)


@pytest.mark.parametrize("n,mode", [(4, "lognormal"), (3, "pow2")])
def test_scaled_shards_merge_to_the_global_selection(n, mode):
    """Scaled keys: each range's selection equals the oracle's ranking of
    that range, and the merge of the shard lists equals the one-device
    scaled Top-K, values included."""
    from test_gpu_scaled import _store_scales
    wl = gen.WORKLOADS["b128_rag"].with_(B=6, L=60000, L_min=2000, D=128, H=16, Di=64)
    log(f"shard scaled n={n} mode={mode}")
    gc = GpuCache(wl, keep_kv=False)
    ks, scales = _store_scales(gc, mode)
    K = 1500
    B, max_ctx = wl.B, int(gc.lens.max())
    q_h = gen.idx_query(wl)
    q = to_dev(q_h)
    bounds = _bounds(max_ctx, n)
    pidx = torch.empty((n, B, K), dtype=torch.int32, device=DEV)
    pval = torch.empty((n, B, K), dtype=torch.float32, device=DEV)
    pcnt = torch.empty((n, B), dtype=torch.int32, device=DEV)
    ws = csa2.Workspace(DEV)
    for s, (a, e) in enumerate(bounds):
        csa2.index_topk_range_scaled(gc.cache, gc.ctx, max_ctx, q, ks, K, a, e, ws,
                                     out_idx=pidx[s], out_count=pcnt[s], out_sel_values=pval[s])
    midx, mcnt, mval = csa2.topk_merge(pidx, pval, pcnt, K, csa2.Workspace(DEV))
    torch.cuda.synchronize()
    pidx, pval, pcnt = to_host(pidx), to_host(pval), to_host(pcnt)
    midx, mcnt, mval = to_host(midx), to_host(mcnt), to_host(mval)
    for b in range(B):
        L = int(gc.lens[b])
        nc = max(0, L - gen.WINDOW)
        v = OS.scaled_values(OS.indexer_scores(q_h[b], gc.keys[b][:nc]), scales[b][:nc])
        for s, (a, e) in enumerate(bounds):
            pos = np.arange(a, min(e, nc)) if min(e, nc) > a else np.zeros(0, np.int64)
            c = min(K, pos.size)
            want = np.sort(pos[OS.rank_order_values(v[pos], pos)[:c]])
            assert int(pcnt[s, b]) == c, f"shard {s} count b={b}"
            assert np.array_equal(pidx[s, b, :c], want), f"shard {s} positions b={b}"
            assert np.array_equal(pval[s, b, :c].view(np.uint32), v[want].view(np.uint32))
        want, wcnt, wval = OS.topk_values(v, L, K)
        assert int(mcnt[b]) == wcnt and np.array_equal(midx[b], want), f"merge b={b}"
        assert np.array_equal(mval[b].view(np.uint32), wval.view(np.uint32)), f"merge values b={b}"
