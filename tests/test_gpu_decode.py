"""GPU parity of csa2_sparse_decode against the fp64 oracle: outputs and LSE
within max-abs 2e-3 on small shapes, for every split plan (one block per
sequence and head group, and many splits merged by the LSE combine), the
degenerate token sets (window only, context shorter than the window, empty
context, every candidate selected -- checked against the oracle's dense
path too), sharp softmax variants, and a crafted cache that holds every
E2M1 code under every E4M3 scale.  Full-size workloads are in
test_gpu_configs.py."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen
from oracle import attention as OA
from oracle import cache as OC
from oracle import formats as OF

from gpu_common import (ATOL, DEV, GpuCache, assert_close, decode_plan, log, oracle_decode,
                        oracle_topk, to_dev, to_host)

pytestmark = pytest.mark.gpu


def _decode_and_check(gc: GpuCache, K: int, layer: int = 0, check_dense: bool = False,
                      plan: str = "auto"):
    wl = gc.wl
    qi = gen.idx_query(wl, layer)
    ws_t, ws_d = csa2.Workspace(DEV), csa2.Workspace(DEV)
    max_ctx = max(1, int(gc.lens.max()))
    idx, cnt = csa2.index_topk(gc.cache, gc.ctx, max_ctx, to_dev(qi), K, ws_t)
    q = gen.query(wl, layer)
    sigma = float(gen.softmax_scale(wl))
    with decode_plan(plan):
        out, lse = csa2.sparse_decode(gc.cache, gc.ctx, to_dev(q), sigma, idx, cnt, gc.swa[layer],
                                      ws_d)
    torch.cuda.synchronize()
    idx_h, cnt_h, out_h, lse_h = to_host(idx), to_host(cnt), to_host(out), to_host(lse)
    worst = 0.0
    for b in range(wl.B):
        L = int(gc.lens[b])
        _, want_idx, wcnt = oracle_topk(gc.keys[b], qi[b], L, K)
        assert int(cnt_h[b]) == wcnt and np.array_equal(idx_h[b], want_idx), f"indices b={b}"
        sel = want_idx[:wcnt]
        o, l = oracle_decode(q[b], sigma, gc.kv_rows(b, sel), gc.rings[layer, b], sel, L)
        worst = max(worst, assert_close(out_h[b], o, ATOL, f"out b={b}"))
        if L == 0:
            assert np.all(np.isneginf(lse_h[b]))
        else:
            assert_close(lse_h[b], l, ATOL, f"lse b={b}")
        if check_dense:
            n = max(0, L - 128)
            x = np.concatenate([OF.dequantize_rows(*OF.quantize_rows(gc.kv[b][:n])),
                                OF.bf16_value(gc.kv[b][n:L])])
            assert_close(out_h[b], OA.dense_reference(q[b], sigma, x), ATOL, f"dense b={b}")
    log(f"  max-abs error {worst:.2e}")
    return worst


def test_tiny():
    log("decode tiny")
    _decode_and_check(GpuCache(gen.WORKLOADS["tiny"]), 256)


@pytest.mark.parametrize("L", [0, 1, 100, 128, 129, 300])
def test_window_heavy_short_contexts(L):
    log(f"decode short L={L}")
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=L)
    _decode_and_check(GpuCache(wl), 64)


@pytest.mark.parametrize("plan", ["hg64", "hg64_split1"])
@pytest.mark.parametrize("L", [0, 1, 100, 129, 300])
def test_window_heavy_short_contexts_h64(L, plan):
    log(f"decode short L={L} H=64 D=512 plan={plan}")
    wl = gen.WORKLOADS["b8_64k"].with_(B=3, L=L)
    _decode_and_check(GpuCache(wl), 64, plan=plan)


def test_all_candidates_equal_dense():
    wl = gen.WORKLOADS["tiny"].with_(L=1500)
    log("decode K = all candidates vs dense")
    _decode_and_check(GpuCache(wl), 1372, check_dense=True)


def test_window_only_K0():
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=3000)
    log("decode K=0 (window only)")
    _decode_and_check(GpuCache(wl), 0)


@pytest.mark.parametrize("plan", ["hg64", "hg64_split3"])
def test_all_candidates_equal_dense_h64(plan):
    wl = gen.WORKLOADS["b8_64k"].with_(B=2, L=1500)
    log(f"decode K = all candidates vs dense, H=64 D=512 plan={plan}")
    _decode_and_check(GpuCache(wl), 1372, check_dense=True, plan=plan)


# (8, 4): logits with a spread of ~46 in log2 units, so later tiles often pass
# the running reference by more than 2^8 and the accumulators are rescaled
@pytest.mark.parametrize("q_std,mult", [(1.0, 1.0), (1.0, 4.0), (8.0, 4.0)])
def test_sharp_softmax(q_std, mult):
    wl = gen.WORKLOADS["tiny"].with_(q_std=q_std, sigma_mult=mult)
    log(f"decode sharp q_std={q_std} sigma x{mult}")
    _decode_and_check(GpuCache(wl), 256)


@pytest.mark.parametrize("plan", ["auto", "hg64", "hg64_split3", "hg64_split1", "hg16_split2"])
@pytest.mark.parametrize("B", [1, 3, 64])
@pytest.mark.parametrize("q_std", [None, 8.0])
def test_d512_h64_split_plans(B, q_std, plan):
    """Every plan on every batch size: 16- and 64-head blocks, one block per
    (sequence, head group) over all tiles, or token splits (1, 2, 3 tiles or
    the library's choice) merged by the combine kernel."""
    wl = gen.WORKLOADS["b8_64k"].with_(B=B, L=4096 + 128 + 37, q_std=q_std)
    log(f"decode D=512 H=64 B={B} q_std={q_std} plan={plan}")
    _decode_and_check(GpuCache(wl), 2048, plan=plan)


@pytest.mark.parametrize("plan", ["auto", "hg64", "hg16_split2"])
@pytest.mark.parametrize("B,H,D,K,lmin,lmax,paged", [
    (64, 64, 512, 256, 0, 700, True),      # ragged, L < 128, counts below K, empty contexts
    (64, 128, 512, 512, 900, 1500, False),  # two 64-head or eight 16-head groups per sequence
    (96, 64, 256, 300, 200, 1200, True),    # K not a multiple of the tile
    (64, 64, 128, 1024, 1100, 1400, False), # K >= candidates for some sequences
])
def test_large_batch_ragged(B, H, D, K, lmin, lmax, paged, plan):
    """Large batches: one block per (sequence, head group) over all of a
    sequence's tiles, or token splits; ragged and paged contexts, empty and
    window-only ones, counts below K."""
    wl = gen.WORKLOADS["tiny"].with_(B=B, H=H, D=D, Di=64, L=lmax, L_min=lmin, ragged=True,
                                     paged=paged)
    log(f"decode large batch B={B} H={H} D={D} K={K} L in [{lmin}, {lmax}] paged={paged} "
        f"plan={plan}")
    _decode_and_check(GpuCache(wl), K, plan=plan)


@pytest.mark.parametrize("plan", ["auto", "hg16_split2"])
@pytest.mark.parametrize("q_std,mult", [(1.0, 1.0), (1.0, 4.0), (8.0, 4.0)])
def test_large_batch_sharp(q_std, mult, plan):
    wl = gen.WORKLOADS["b8_64k"].with_(B=64, L=3000, q_std=q_std, sigma_mult=mult)
    log(f"decode large batch sharp q_std={q_std} sigma x{mult} plan={plan}")
    _decode_and_check(GpuCache(wl), 2048, plan=plan)


@pytest.mark.parametrize("plan", ["auto", "hg64", "hg16_split4", "hg64_split5"])
@pytest.mark.parametrize("D,H", [(256, 32), (128, 128), (256, 64)])
def test_other_widths(D, H, plan):
    """Latent widths 256 and 128; with 4 splits of 16-head blocks or 2 of
    64-head ones the combine takes several float4s per thread."""
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=2000, D=D, H=H, Di=128)
    log(f"decode D={D} H={H} plan={plan}")
    _decode_and_check(GpuCache(wl), 512, plan=plan)


@pytest.mark.parametrize("H,plan", [(16, "auto"), (64, "hg64"), (64, "hg64_split3")])
def test_every_code_under_every_scale(H, plan):
    """512 crafted rows: group g of row r has scale code (32r+g) % 127 and code
    bytes cycling through all 256 values, so every (E2M1 code, E4M3 scale)
    pair is dequantised.  q = 0 makes the output the plain mean of all rows;
    the window ring is zero.  fp32 summation of 512 rows of magnitude <= 2688,
    divided by 640 rows, stays below 2e-4."""
    D, Di, n_sel = 512, 128, 512
    L = n_sel + 128
    mp = L // 64
    pt = np.arange(mp, dtype=np.int32)[None, :]
    pages = np.zeros((mp, OC.page_bytes(D, Di)), np.uint8)
    r = np.arange(L)[:, None]
    g = np.arange(D // 16)[None, :]
    scales = ((32 * r + g) % 127).astype(np.uint8)
    codes = ((r * D // 2 + np.arange(D // 2)[None, :]) % 256).astype(np.uint8)
    R = D // 2 + D // 16                      # a row: its codes, then its scales
    for p in range(L):
        pg, row = p // 64, p % 64
        pages[pg, row * R:row * R + D // 2] = codes[p]
        pages[pg, row * R + D // 2:(row + 1) * R] = scales[p]
    cache = csa2.Cache(to_dev(pages), to_dev(pt), D, Di)
    ctx = to_dev(np.array([L], np.int32))
    idx = to_dev(np.arange(n_sel, dtype=np.int32)[None, :])
    cnt = to_dev(np.array([n_sel], np.int32))
    swa = torch.zeros((1, 128, D), dtype=torch.uint16, device=DEV)
    q = torch.zeros((1, H, D), dtype=torch.uint16, device=DEV)
    with decode_plan(plan):
        out, lse = csa2.sparse_decode(cache, ctx, q, 0.1, idx, cnt, swa, csa2.Workspace(DEV))
    torch.cuda.synchronize()
    x = np.concatenate([OF.dequantize_rows(codes[:n_sel], scales[:n_sel]), np.zeros((128, D))])
    want = np.repeat(x.mean(0)[None, :], H, 0)
    err = assert_close(to_host(out)[0], want, 2e-4, "mean of crafted rows")
    assert_close(to_host(lse)[0], np.full(H, np.log(L)), 1e-5, "lse")
    log(f"  crafted dequant sweep H={H} plan={plan} max-abs error {err:.2e}")


def test_invalid_indices_are_masked():
    """Entries inside the window range, beyond the context or negative are
    skipped (no memory access outside the cache); the rest decodes normally."""
    wl = gen.WORKLOADS["tiny"].with_(L=1000)
    gc = GpuCache(wl)
    good = np.array([3, 50, 400, 871], np.int32)
    bad = np.array([-5, 872, 999, 1 << 30], np.int32)
    idx = np.concatenate([good, bad])[None, :]
    q = gen.query(wl)
    sigma = float(gen.softmax_scale(wl))
    out, _ = csa2.sparse_decode(gc.cache, gc.ctx, to_dev(q), sigma, to_dev(idx),
                                to_dev(np.array([8], np.int32)), gc.swa[0], csa2.Workspace(DEV))
    torch.cuda.synchronize()
    o, _ = oracle_decode(q[0], sigma, gc.kv_rows(0, good), gc.rings[0, 0], good, 1000)
    assert_close(to_host(out)[0], o, ATOL, "masked invalid entries")
