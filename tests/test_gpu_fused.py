"""GPU parity of csa2_append_index_topk: a decode append fused into the Full
layer's scoring launch must give, bit for bit, what csa2_quantize_append
followed by csa2_index_topk gives (pages, window ring, scores, indices,
counts), and the indices must match the oracle.  A token at a scoring
candidate position is not written by the fused call."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen

from gpu_common import DEV, GpuCache, log, oracle_topk, to_dev, to_host

pytestmark = pytest.mark.gpu


def _twin(gc: GpuCache):
    """A second cache and ring with the same bytes as gc's."""
    wl = gc.wl
    cache = csa2.Cache(gc.cache.pages.clone(), gc.cache.page_table, wl.D, wl.Di)
    return cache, gc.swa[0].clone()


def _tokens(wl, lens, per_seq: int, step0: int):
    """per_seq new tokens per sequence at positions L_b, L_b + 1, ..."""
    xs, ks, seq, pos = [], [], [], []
    for t in range(per_seq):
        x, k = gen.append_tokens(wl, step0 + t)
        xs.append(x)
        ks.append(k)
        seq.append(np.arange(wl.B, dtype=np.int32))
        pos.append((lens + t).astype(np.int32))
    return (np.concatenate(xs), np.concatenate(ks), np.concatenate(seq), np.concatenate(pos))


def _run_pair(gc: GpuCache, per_seq: int, K: int, stray: bool):
    wl = gc.wl
    lens = gc.lens
    x, k, seq, pos = _tokens(wl, lens, per_seq, 0)
    new_lens = (lens + per_seq).astype(np.int32)
    keep = np.ones(len(seq), bool)
    if stray:
        # a token of sequence 0 aimed at a scoring candidate (position 5)
        xs, ks = gen.append_tokens(wl, 100)
        x = np.concatenate([x, xs[:1]])
        k = np.concatenate([k, ks[:1]])
        seq = np.concatenate([seq, [0]]).astype(np.int32)
        pos = np.concatenate([pos, [5]]).astype(np.int32)
        keep = np.concatenate([keep, [new_lens[0] - 128 <= 5]])
    ctx = to_dev(new_lens)
    max_ctx = int(new_lens.max())
    ref_cache, ref_ring = _twin(gc)

    # reference: the two calls, with only the tokens the fused call writes
    csa2.quantize_append(ref_cache, to_dev(x[keep]), to_dev(seq[keep]), to_dev(pos[keep]),
                         keys=to_dev(k[keep]), swa=ref_ring)
    ref_scores = torch.full((wl.B, max_ctx), -7, dtype=torch.int32, device=DEV)
    ref_idx, ref_cnt = csa2.index_topk(ref_cache, ctx, max_ctx, to_dev(gen.idx_query(wl)), K,
                                       csa2.Workspace(DEV), out_scores=ref_scores)
    # fused
    scores = torch.full((wl.B, max_ctx), -7, dtype=torch.int32, device=DEV)
    idx, cnt = csa2.append_index_topk(gc.cache, to_dev(x), to_dev(seq), to_dev(pos), to_dev(k),
                                      gc.swa[0], ctx, max_ctx, to_dev(gen.idx_query(wl)), K,
                                      csa2.Workspace(DEV), out_scores=scores)
    torch.cuda.synchronize()
    assert torch.equal(gc.cache.pages, ref_cache.pages), "pages differ"
    assert torch.equal(gc.swa[0], ref_ring), "window rings differ"
    assert torch.equal(scores, ref_scores), "scores differ"
    assert torch.equal(idx, ref_idx) and torch.equal(cnt, ref_cnt), "selection differs"
    idx, cnt = to_host(idx), to_host(cnt)
    for b in range(wl.B):
        _, want, wcnt = oracle_topk(gc.keys[b], gen.idx_query(wl)[b], int(new_lens[b]), K)
        assert int(cnt[b]) == wcnt and np.array_equal(idx[b], want), f"oracle b={b}"


@pytest.mark.parametrize("per_seq,stray", [(1, False), (3, True)])
def test_tiny(per_seq, stray):
    wl = gen.WORKLOADS["tiny"].with_(B=3, L=5000, append_steps=4)
    log(f"fused append+topk tiny per_seq={per_seq} stray={stray}")
    _run_pair(GpuCache(wl, keep_kv=False), per_seq, 256, stray)


def test_paged_ragged_d512():
    wl = gen.WORKLOADS["b128_rag"].with_(B=12, L=40000, L_min=1)
    log("fused append+topk paged ragged B=12 D=512")
    _run_pair(GpuCache(wl, keep_kv=False), 1, 2048, True)


def test_many_block_scoring_grid():
    """The fused call on a grid of 8-page scoring blocks (40 sequences of
    100K-110K positions)."""
    wl = gen.WORKLOADS["b128_rag"].with_(B=40, L=110_000, L_min=100_000, D=128, H=16)
    log("fused append+topk many-block scoring grid")
    _run_pair(GpuCache(wl, keep_kv=False), 1, 2048, True)


def test_b8_64k_shape():
    wl = gen.WORKLOADS["b8_64k"].with_(append_steps=1)
    log("fused append+topk b8_64k")
    _run_pair(GpuCache(wl, keep_kv=False), 1, wl.K, False)
