"""End-to-end GPU parity on the five workloads at their full sizes.

Indices (and their counts) bit-exact against the oracle for every sequence
and layer; the stored FP4 codes and E4M3 scales of every selected row
bit-exact against the oracle's quantisation of the same bf16 draw; attention
outputs within max-abs 2e-3 and LSE within 2e-3 of the fp64 oracle, for every
sequence.  Whole pages are compared too: all pages of two b8_64k sequences,
and every page the b128_rag append writes into.

  tiny       B=1, L=4096, H=16, D=128, Di=64, K=256
  b8_64k     B=8, L=65536, H=64, D=512, Di=128, K=2048
  chain_64k  the same cache and shapes, Full (pool 8192) -> Reindex (2048) -> Reuse
  b1_1m      B=1, L=2^20, K=2048, 1% of keys boosted towards the query
  b128_rag   B=128, L ~ U{8192..131072}, permuted 64-token pages, one appended
             token per sequence before the decode step
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen
from oracle import attention as OA
from oracle import cache as OC
from oracle import formats as OF
from oracle import select as OS

from gpu_common import (ATOL, DEV, THREADS, GpuCache, assert_close, log, oracle_topk, to_dev,
                        to_host)

pytestmark = pytest.mark.gpu


def stored_rows(gc, b: int, sel: np.ndarray):
    """The GPU cache's codes [n, D/2] and scales [n, D/16] of positions sel of
    sequence b, gathered on the GPU by the documented page layout."""
    wl = gc.wl
    ci, si = OC.row_byte_index(gc.pt, wl.D, wl.Di, b, sel)
    flat = gc.cache.pages.view(-1)
    return (to_host(flat[to_dev(ci.reshape(-1))]).reshape(ci.shape),
            to_host(flat[to_dev(si.reshape(-1))]).reshape(si.shape))


def check_selected(gc, b: int, q_bits, sigma, sel, L, ring, out_b, lse_b, what: str) -> float:
    """Stored FP4 bytes of the selected rows bit-exact against the oracle's
    quantisation of their bf16 draw, then attention within ATOL."""
    codes, scales = OF.quantize_rows(gc.kv_rows(b, sel)) if len(sel) else (
        np.zeros((0, gc.wl.D // 2), np.uint8), np.zeros((0, gc.wl.D // 16), np.uint8))
    gcodes, gscales = stored_rows(gc, b, sel)
    assert np.array_equal(gcodes, codes), f"{what}: FP4 codes of selected rows, b={b}"
    assert np.array_equal(gscales, scales), f"{what}: E4M3 scales of selected rows, b={b}"
    o, l = OA.sparse_decode(q_bits, sigma, codes, scales, ring, sel, L)
    err = assert_close(out_b, o, ATOL, f"{what} out b={b}")
    assert_close(lse_b, l, ATOL, f"{what} lse b={b}")
    return err


def _full_layer(gc, K, layer=0):
    wl = gc.wl
    qi, q = gen.idx_query(wl, layer), gen.query(wl, layer)
    sigma = float(gen.softmax_scale(wl))
    max_ctx = int(gc.lens.max())
    idx, cnt = csa2.index_topk(gc.cache, gc.ctx, max_ctx, to_dev(qi), K, csa2.Workspace(DEV))
    out, lse = csa2.sparse_decode(gc.cache, gc.ctx, to_dev(q), sigma, idx, cnt, gc.swa[layer],
                                  csa2.Workspace(DEV))
    torch.cuda.synchronize()
    idx_h, cnt_h, out_h, lse_h = map(to_host, (idx, cnt, out, lse))

    def one(b):
        L = int(gc.lens[b])
        _, want, wcnt = oracle_topk(gc.keys[b], qi[b], L, K)
        assert int(cnt_h[b]) == wcnt and np.array_equal(idx_h[b], want), f"indices b={b}"
        sel = want[:wcnt]
        return check_selected(gc, b, q[b], sigma, sel, L, gc.rings[layer, b], out_h[b], lse_h[b],
                              wl.name)

    with ThreadPoolExecutor(THREADS) as ex:
        worst = max(ex.map(one, range(wl.B)))
    log(f"  {wl.name}: indices and selected FP4 rows bit-exact for {wl.B} sequences; "
        f"max-abs output error {worst:.2e}")
    return idx, cnt


def assert_pages_equal(gc, b: int, L: int, kv: np.ndarray, keys: np.ndarray, what: str) -> None:
    """Every page holding positions [0, L) of sequence b, byte for byte, against
    the oracle's append of the same draw (rows past L are zero on both sides)."""
    wl = gc.wl
    n_pg = -(-L // 64)
    pids = gc.pt[b, :n_pg]
    got = to_host(gc.cache.pages[to_dev(pids.astype(np.int64))])
    want = np.zeros_like(got)
    local = np.arange(n_pg, dtype=np.int32)[None, :]
    chunk = 8192

    def part(lo):
        hi = min(L, lo + chunk)
        OC.append(want, local, wl.D, wl.Di, np.zeros(hi - lo, int), np.arange(lo, hi), kv[lo:hi],
                  keys[lo:hi], None)

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(part, range(0, L, chunk)))
    assert np.array_equal(got, want), f"{what}: pages of sequence {b}"


def test_tiny_full():
    log("config tiny")
    _full_layer(GpuCache(gen.WORKLOADS["tiny"]), 256)


def test_b8_64k_full():
    log("config b8_64k")
    gc = GpuCache(gen.WORKLOADS["b8_64k"])
    for b in (0, 7):
        assert_pages_equal(gc, b, int(gc.lens[b]), gc.kv[b], gc.keys[b], "b8_64k")
    log("  b8_64k: all 2 x 1024 pages of sequences 0 and 7 bit-exact")
    _full_layer(gc, 2048)


def test_b1_1m_full():
    log("config b1_1m")
    gc = GpuCache(gen.WORKLOADS["b1_1m"])
    _full_layer(gc, 2048)


def test_chain_64k_full():
    wl = gen.WORKLOADS["chain_64k"]
    log("config chain_64k")
    gc = GpuCache(wl, layers=3)
    sigma = float(gen.softmax_scale(wl))
    q_idx = [gen.idx_query(wl, i) for i in range(2)]
    qs = [gen.query(wl, i) for i in range(3)]
    # Full layer: pool of 8192 + its own window
    pool, pc = _full_layer(gc, wl.K, layer=0)
    # Reindex layer: refilter the pool to 2048 with its own indexer query
    idx, cnt = csa2.reindex(gc.cache, to_dev(q_idx[1]), pool, pc, wl.K2, csa2.Workspace(DEV))
    outs = [csa2.sparse_decode(gc.cache, gc.ctx, to_dev(qs[i]), sigma, idx, cnt, gc.swa[i],
                               csa2.Workspace(DEV)) for i in (1, 2)]     # Reindex, Reuse
    torch.cuda.synchronize()
    idx_h, cnt_h = to_host(idx), to_host(cnt)
    worst = 0.0
    for b in range(wl.B):
        L = int(gc.lens[b])
        _, opool, opc = oracle_topk(gc.keys[b], q_idx[0][b], L, wl.K)     # the oracle's own pool
        p = opool[:opc]
        want, wcnt = OS.reindex(opool, opc, OS.indexer_scores(q_idx[1][b], gc.keys[b][p]), wl.K2)
        assert int(cnt_h[b]) == wcnt and np.array_equal(idx_h[b], want), f"reindex b={b}"
        sel = want[:wcnt]
        for layer, (out, lse) in zip((1, 2), outs):
            worst = max(worst, check_selected(gc, b, qs[layer][b], sigma, sel, L,
                                              gc.rings[layer, b], to_host(out)[b],
                                              to_host(lse)[b], f"chain layer {layer}"))
    log(f"  chain: Reindex/Reuse indices bit-exact; max-abs output error {worst:.2e}")


def test_b128_ragged_append_step():
    wl = gen.WORKLOADS["b128_rag"]
    log("config b128_rag: building the paged cache")
    gc = GpuCache(wl, keep_kv=False)
    # decode step: one new token per sequence at position L_b, written into the
    # FP4 cache, the indexer keys and the window ring, then select and attend
    x, k = gen.append_tokens(wl, 0)
    pos = gc.lens.astype(np.int32)
    csa2.quantize_append(gc.cache, to_dev(x), torch.arange(wl.B, dtype=torch.int32, device=DEV),
                         to_dev(pos), keys=to_dev(k), swa=gc.swa[0])
    new_lens = gc.lens + 1
    gc.ctx = to_dev(new_lens.astype(np.int32))
    for b in range(wl.B):
        gc.keys[b] = np.concatenate([gc.keys[b], k[b:b + 1]])
        gc.rings[0, b, pos[b] % 128] = x[b]
    gc.lens = new_lens
    ring_gpu = to_host(gc.swa[0])
    assert np.array_equal(ring_gpu, gc.rings[0]), "window rings after append"

    def rows(b, sel):      # rows of the grown sequences: the draw plus the appended token
        sel = np.asarray(sel)
        out = np.empty((sel.size, wl.D), np.uint16)
        old = sel < pos[b]
        if old.any():
            out[old] = gen.kv_bf16(wl, b, int(pos[b]))[sel[old]]
        out[~old] = x[b]
        return out

    gc.kv_rows = rows
    # every page the append wrote into, whole: the bulk-filled rows before the
    # new token, the new token's row and key, zeros after it
    pg_new = gc.pt[np.arange(wl.B), pos // 64]
    got = to_host(gc.cache.pages[to_dev(pg_new.astype(np.int64))])

    def page(b):
        lo = int(pos[b]) // 64 * 64
        want = np.zeros((1, got.shape[1]), np.uint8)
        kv_b = rows(b, np.arange(lo, int(pos[b]) + 1))
        OC.append(want, np.zeros((1, gc.pt.shape[1]), np.int32), wl.D, wl.Di,
                  np.zeros(kv_b.shape[0], int), np.arange(lo, int(pos[b]) + 1) - lo,
                  kv_b, gc.keys[b][lo:int(pos[b]) + 1], None)
        assert np.array_equal(got[b], want[0]), f"appended page of sequence {b}"

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(page, range(wl.B)))
    log(f"  b128_rag: the {wl.B} pages the append wrote into are bit-exact")
    _full_layer(gc, wl.K)
