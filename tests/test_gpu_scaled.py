"""GPU parity of the scaled indexer (csa2_store_key_scales,
csa2_index_topk_scaled, csa2_reindex_scaled) against the oracle.

The oracle ranks v_p = fl32(s_p * score_p) (value descending, position
ascending, -0 equal to +0).  Everything is compared bit for bit: the stored
scale array, every value, the selected positions and their values.  Cases:
the one-block plan over every K edge, scale draws that force exact ties
(powers of two, signed with zeros), values that differ only in their lowest
mantissa bits (the third radix digit decides), subnormal products,
candidates past the on-chip lists, the multi-block plan with its direct and
general final stages, a paged ragged batch, and Reindex over a scaled pool."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen
from oracle import formats as OF
from oracle import select as OS

from gpu_common import DEV, GpuCache, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _store_scales(gc: GpuCache, mode: str) -> tuple[torch.Tensor, list]:
    """Key scales of every cached position, written through the page table."""
    ks = csa2.key_scales_for(gc.cache)
    host = []
    for b in range(gc.wl.B):
        L = int(gc.lens[b])
        s = gen.key_scales(gc.wl, b, L, mode)
        host.append(s)
        if L > 0:
            csa2.store_key_scales(gc.cache, to_dev(s),
                                  torch.full((L,), b, dtype=torch.int32, device=DEV),
                                  torch.arange(L, dtype=torch.int32, device=DEV), ks)
    torch.cuda.synchronize()
    return ks, host


def _oracle_values(gc: GpuCache, q: np.ndarray, scales: list, b: int) -> np.ndarray:
    n = max(0, int(gc.lens[b]) - gen.WINDOW)
    sc = OS.indexer_scores(q[b], gc.keys[b][:n])
    return OS.scaled_values(sc, scales[b][:n])


def _check_topk(gc: GpuCache, q: np.ndarray, ks: torch.Tensor, scales: list, K: int,
                ws=None):
    wl = gc.wl
    max_ctx = int(gc.lens.max())
    vals = torch.full((wl.B, max_ctx), float("nan"), dtype=torch.float32, device=DEV)
    sel = torch.full((wl.B, K), float("nan"), dtype=torch.float32, device=DEV)
    idx, cnt, _ = csa2.index_topk_scaled(gc.cache, gc.ctx, max_ctx, to_dev(q), ks, K,
                                         ws or csa2.Workspace(DEV), out_values=vals,
                                         out_sel_values=sel)
    torch.cuda.synchronize()
    idx, cnt, vals, sel = to_host(idx), to_host(cnt), to_host(vals), to_host(sel)
    for b in range(wl.B):
        L = int(gc.lens[b])
        v = _oracle_values(gc, q, scales, b)
        want, wcnt, wsel = OS.topk_values(v, L, K)
        n = v.size
        assert np.array_equal(vals[b, :n].view(np.uint32), v.view(np.uint32)), \
            f"values differ, b={b}"
        assert int(cnt[b]) == wcnt, f"count b={b}: {cnt[b]} vs {wcnt}"
        assert np.array_equal(idx[b], want), f"indices differ, b={b}"
        assert np.array_equal(sel[b].view(np.uint32), wsel.view(np.uint32)), \
            f"selected values differ, b={b}"
    return idx, cnt


def _same_row_keys(b, k):
    """Every key equal to row 0: one score for all positions, so the order is
    decided by the scales alone."""
    out = k.copy()
    out[:] = k[0]
    return out


def test_store_key_scales_layout():
    wl = gen.WORKLOADS["b128_rag"].with_(B=5, L=3000, L_min=1, D=128, H=16, Di=64)
    log("scaled store layout")
    gc = GpuCache(wl, keep_kv=False)
    ks, host = _store_scales(gc, "lognormal")
    got = to_host(ks)
    want = np.zeros_like(got)
    for b in range(wl.B):
        L = int(gc.lens[b])
        p = np.arange(L)
        want[gc.pt[b, p // gen.PAGE], p % gen.PAGE] = host[b]
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("K", [0, 1, 2, 255, 256, 3967, 3968, 5000])
def test_tiny_all_K(K):
    wl = gen.WORKLOADS["tiny"]
    log(f"scaled tiny K={K}")
    gc = GpuCache(wl)
    ks, scales = _store_scales(gc, "lognormal")
    _check_topk(gc, gen.idx_query(wl), ks, scales, K)


@pytest.mark.parametrize("mode", ["pow2", "signed", "fine", "subnormal"])
def test_scale_modes(mode):
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=6000)
    log(f"scaled modes mode={mode}")
    gc = GpuCache(wl, keys_fn=_same_row_keys if mode == "fine" else None)
    ks, scales = _store_scales(gc, mode)
    q = gen.idx_query(wl)
    for K in (1, 100, 777, 2048, 5871):
        _check_topk(gc, q, ks, scales, K)


@pytest.mark.parametrize("mode", ["fine", "pow2"])
def test_ties_past_the_lds_candidate_list(mode):
    """~16K candidates with one score: every candidate shares the top digit,
    more than the one-block selection keeps on chip."""
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=16000)
    log(f"scaled one score L=16000 mode={mode}")
    gc = GpuCache(wl, keys_fn=_same_row_keys)
    ks, scales = _store_scales(gc, mode)
    q = gen.idx_query(wl)
    for K in (2048, 7000, 15000):
        _check_topk(gc, q, ks, scales, K)


@pytest.mark.parametrize("mode,L,Ks", [
    ("lognormal", 65536 + 128, (2048, 8192)),      # direct final stage (<= 16 chunks)
    ("lognormal", 150_000, (2048, 65536)),         # general final stage, list overflow
    ("fine", 70_000, (2048, 30000)),               # one score: third digit, general stage
])
def test_multi_block_plan(mode, L, Ks):
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=L, Di=64)
    log(f"scaled multi-block L={L} mode={mode}")
    gc = GpuCache(wl, keep_kv=False, keys_fn=_same_row_keys if mode == "fine" else None)
    ks, scales = _store_scales(gc, mode)
    q = gen.idx_query(wl)
    for K in Ks:
        _check_topk(gc, q, ks, scales, K)


def test_paged_ragged_batch_and_workspace_reuse():
    wl = gen.WORKLOADS["b128_rag"].with_(B=16, L=40000, L_min=1, D=128, H=16)
    log("scaled paged ragged B=16")
    gc = GpuCache(wl, keep_kv=False)
    ks, scales = _store_scales(gc, "signed")
    q = gen.idx_query(wl)
    ws = csa2.Workspace(DEV)
    a = _check_topk(gc, q, ks, scales, 512, ws=ws)
    b = _check_topk(gc, q, ks, scales, 512, ws=ws)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    # the int32 path on the same workspace afterwards is unaffected
    idx, cnt = csa2.index_topk(gc.cache, gc.ctx, int(gc.lens.max()), to_dev(q), 512, ws)
    torch.cuda.synchronize()
    for bb in range(wl.B):
        sc = OS.indexer_scores(q[bb], gc.keys[bb][:max(0, int(gc.lens[bb]) - gen.WINDOW)])
        want, _ = OS.topk(sc, int(gc.lens[bb]), 512)
        assert np.array_equal(to_host(idx)[bb], want)


@pytest.mark.parametrize("mode,K_full,K2", [("lognormal", 4096, 512), ("fine", 20000, 3000),
                                             ("signed", 1000, 1000), ("fine", 8191, 2000),
                                             ("lognormal", 12290, 3000)])
def test_reindex_scaled(mode, K_full, K2):
    """Full layer (scaled) builds the pool; a Reindex layer with its own
    query ranks the pool entries by their scaled values."""
    wl = gen.WORKLOADS["tiny"].with_(B=3, L=40000, Di=64)
    log(f"scaled reindex mode={mode} K_full={K_full} K2={K2}")
    gc = GpuCache(wl, keep_kv=False, keys_fn=_same_row_keys if mode == "fine" else None)
    ks, scales = _store_scales(gc, mode)
    q0 = gen.idx_query(wl, 0)
    q1 = gen.idx_query(wl, 1)
    pool, pcnt = _check_topk(gc, q0, ks, scales, K_full)
    vals = torch.full((wl.B, K_full), float("nan"), dtype=torch.float32, device=DEV)
    idx, cnt = csa2.reindex_scaled(gc.cache, to_dev(q1), ks, to_dev(pool), to_dev(pcnt), K2,
                                   csa2.Workspace(DEV), out_values=vals)
    torch.cuda.synchronize()
    idx, cnt, vals = to_host(idx), to_host(cnt), to_host(vals)
    for b in range(wl.B):
        c = int(pcnt[b])
        p = pool[b, :c]
        v = OS.scaled_values(OS.indexer_scores(q1[b], gc.keys[b][p]), scales[b][p])
        assert np.array_equal(vals[b, :c].view(np.uint32), v.view(np.uint32)), f"b={b}"
        want, wcnt = OS.reindex_values(pool[b], c, v, K2)
        assert int(cnt[b]) == wcnt and np.array_equal(idx[b], want), f"b={b}"


@pytest.mark.parametrize("Di", [64, 128])
def test_many_block_scoring_grid(Di):
    """Scaled keys on a grid of 8-page scoring blocks (40 sequences of
    100K-110K positions)."""
    wl = gen.WORKLOADS["b128_rag"].with_(B=40, L=110_000, L_min=100_000, D=128, H=16, Di=Di)
    log(f"scaled many-block scoring grid Di={Di}")
    gc = GpuCache(wl, keep_kv=False)
    ks, scales = _store_scales(gc, "lognormal")
    _check_topk(gc, gen.idx_query(wl), ks, scales, 2048)


def test_e4m3_scales():
    """E4M3 scale bytes: stored as their exact fp32 values, then ranked."""
    wl = gen.WORKLOADS["b128_rag"].with_(B=6, L=30000, L_min=1, D=128, H=16, Di=64)
    log("scaled e4m3 store + topk")
    gc = GpuCache(wl, keep_kv=False)
    ks = csa2.key_scales_for(gc.cache)
    scales = []
    want = np.zeros(tuple(ks.shape), np.float32)
    for b in range(wl.B):
        L = int(gc.lens[b])
        codes = gen.key_scales_e4m3(wl, b, L)
        s = OF.e4m3_value(codes).astype(np.float32)     # exact: E4M3 values are float32 values
        scales.append(s)
        p = np.arange(L)
        want[gc.pt[b, p // gen.PAGE], p % gen.PAGE] = s
        if L > 0:
            csa2.store_key_scales(gc.cache, to_dev(codes),
                                  torch.full((L,), b, dtype=torch.int32, device=DEV),
                                  torch.arange(L, dtype=torch.int32, device=DEV), ks)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ks).view(np.uint32), want.view(np.uint32))
    q = gen.idx_query(wl)
    for K in (1, 300, 4000):
        _check_topk(gc, q, ks, scales, K)


def test_b8_64k_scaled():
    """The headline shape with scaled keys: every sequence checked in full."""
    wl = gen.WORKLOADS["b8_64k"]
    log("scaled b8_64k")
    gc = GpuCache(wl, keep_kv=False)
    ks, scales = _store_scales(gc, "lognormal")
    _check_topk(gc, gen.idx_query(wl), ks, scales, wl.K)


def test_non_finite_scales_keep_the_output_well_formed():
    """Non-finite scales give an unspecified order, never a fault: the output
    is still count = min(K, n) distinct candidate positions, ascending, -1
    padded."""
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=30000, Di=64)
    log("scaled non-finite scales")
    gc = GpuCache(wl, keep_kv=False)
    ks, scales = _store_scales(gc, "lognormal")
    bad = []
    for b in range(wl.B):
        L = int(gc.lens[b])
        s = scales[b].copy()
        r = np.random.default_rng(b)
        sel = r.choice(L, size=300, replace=False)
        s[sel[:100]] = np.inf
        s[sel[100:200]] = -np.inf
        s[sel[200:]] = np.nan
        bad.append(s)
        csa2.store_key_scales(gc.cache, to_dev(s), torch.full((L,), b, dtype=torch.int32, device=DEV),
                              torch.arange(L, dtype=torch.int32, device=DEV), ks)
    torch.cuda.synchronize()
    q = gen.idx_query(wl)
    for K in (100, 5000):
        idx, cnt, _ = csa2.index_topk_scaled(gc.cache, gc.ctx, int(gc.lens.max()), to_dev(q), ks,
                                             K, csa2.Workspace(DEV))
        torch.cuda.synchronize()
        idx, cnt = to_host(idx), to_host(cnt)
        for b in range(wl.B):
            n = int(gc.lens[b]) - gen.WINDOW
            c = int(cnt[b])
            assert c == min(K, n)
            got = idx[b, :c]
            assert np.all(np.diff(got) > 0) and got[0] >= 0 and got[-1] < n
            assert np.all(idx[b, c:] == -1)
