"""End-to-end GPU parity on the five workloads at their full sizes.

Indices (and their counts) bit-exact against the oracle for every sequence
and layer; attention outputs within max-abs 2e-3 and LSE within 2e-3 of the
fp64 oracle, for every sequence where the oracle is cheap and on a fixed
sample of sequences for the 128-sequence ragged batch.

  tiny       B=1, L=4096, H=16, D=128, Di=64, K=256
  b8_64k     B=8, L=65536, H=64, D=512, Di=128, K=2048
  chain_64k  the same cache and shapes, Full (pool 8192) -> Reindex (2048) -> Reuse
  b1_1m      B=1, L=2^20, K=2048, 1% of keys boosted towards the query
  b128_rag   B=128, L ~ U{8192..131072}, permuted 64-token pages, one appended
             token per sequence before the decode step
"""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen
from oracle import select as OS

from gpu_common import (ATOL, DEV, GpuCache, assert_close, log, oracle_decode, oracle_topk,
                        to_dev, to_host)

pytestmark = pytest.mark.gpu


def _full_layer(gc, K, layer=0, sample=None):
    wl = gc.wl
    qi, q = gen.idx_query(wl, layer), gen.query(wl, layer)
    sigma = float(gen.softmax_scale(wl))
    max_ctx = int(gc.lens.max())
    idx, cnt = csa2.index_topk(gc.cache, gc.ctx, max_ctx, to_dev(qi), K, csa2.Workspace(DEV))
    out, lse = csa2.sparse_decode(gc.cache, gc.ctx, to_dev(q), sigma, idx, cnt, gc.swa[layer],
                                  csa2.Workspace(DEV))
    torch.cuda.synchronize()
    idx_h, cnt_h, out_h, lse_h = map(to_host, (idx, cnt, out, lse))
    worst = 0.0
    for b in range(wl.B):
        L = int(gc.lens[b])
        _, want, wcnt = oracle_topk(gc.keys[b], qi[b], L, K)
        assert int(cnt_h[b]) == wcnt and np.array_equal(idx_h[b], want), f"indices b={b}"
        if sample is not None and b not in sample:
            continue
        sel = want[:wcnt]
        o, l = oracle_decode(q[b], sigma, gc.kv_rows(b, sel), gc.rings[layer, b], sel, L)
        worst = max(worst, assert_close(out_h[b], o, ATOL, f"out b={b}"))
        assert_close(lse_h[b], l, ATOL, f"lse b={b}")
    log(f"  {wl.name}: indices bit-exact for {wl.B} sequences; max-abs output error {worst:.2e}")
    return idx, cnt


def test_tiny_full():
    log("config tiny")
    _full_layer(GpuCache(gen.WORKLOADS["tiny"]), 256)


def test_b8_64k_full():
    log("config b8_64k")
    _full_layer(GpuCache(gen.WORKLOADS["b8_64k"]), 2048)


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
            o, l = oracle_decode(qs[layer][b], sigma, gc.kv_rows(b, sel), gc.rings[layer, b], sel, L)
            worst = max(worst, assert_close(to_host(out)[b], o, ATOL, f"layer {layer} out b={b}"))
            assert_close(to_host(lse)[b], l, ATOL, f"layer {layer} lse b={b}")
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
    sample = set(np.argsort(gc.lens)[[0, 1, -1, -2]].tolist()) | {3, 17, 42, 64, 99, 127}
    _full_layer(gc, wl.K, sample=sample)
