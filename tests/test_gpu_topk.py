"""GPU parity of csa2_index_topk against the oracle: int32 scores and Top-K
indices bit-exact (ties to the lower position), on small shapes and the edge
cases of the selection (planted ties, all-equal scores, K = 0, K >= number of
candidates, context shorter than the window, kept candidates past the
on-chip lists, long sequences, paged ragged batches, top scores clustered
in a few 1024-position blocks).  Full-size workloads are in
test_gpu_configs.py."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen

from gpu_common import DEV, GpuCache, log, oracle_topk, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(gc: GpuCache, q_idx: np.ndarray, K: int, ws=None, max_ctx=None):
    wl = gc.wl
    max_ctx = int(gc.lens.max()) if max_ctx is None else max_ctx
    ws = ws or csa2.Workspace(DEV)
    scores = torch.full((wl.B, max_ctx), -7, dtype=torch.int32, device=DEV)
    idx, cnt = csa2.index_topk(gc.cache, gc.ctx, max_ctx, to_dev(q_idx), K, ws,
                               out_scores=scores)
    torch.cuda.synchronize()
    return to_host(idx), to_host(cnt), to_host(scores)


def _check(gc: GpuCache, q_idx: np.ndarray, K: int, **kw):
    idx, cnt, scores = _run(gc, q_idx, K, **kw)
    for b in range(gc.wl.B):
        L = int(gc.lens[b])
        sc, want, wcnt = oracle_topk(gc.keys[b], q_idx[b], L, K)
        n = sc.size
        assert np.array_equal(scores[b, :n], sc), f"scores differ, b={b}"
        assert int(cnt[b]) == wcnt, f"count b={b}: {cnt[b]} vs {wcnt}"
        assert np.array_equal(idx[b], want), f"indices differ, b={b}"
    return idx, cnt


@pytest.mark.parametrize("K", [0, 1, 2, 255, 256, 3967, 3968, 5000])
def test_tiny_all_K(K):
    wl = gen.WORKLOADS["tiny"]
    log(f"topk tiny K={K}")
    gc = GpuCache(wl)
    _check(gc, gen.idx_query(wl), K)


@pytest.mark.parametrize("L", [0, 1, 127, 128, 129, 130, 191, 200, 1152, 1153])
def test_short_contexts(L):
    wl = gen.WORKLOADS["tiny"].with_(L=L)
    log(f"topk short L={L}")
    gc = GpuCache(wl)
    _check(gc, gen.idx_query(wl), 16)


@pytest.mark.parametrize("L", [4224, 4225, 12416, 16512, 16513])
def test_one_block_row_boundaries(L):
    """Candidate counts at the one-block selection's load-row edges: 4096
    (one full row), 4097 (one live entry in the second), 12288, 16384 (the
    largest one-block case, four full rows) and 16385 (the filter plan)."""
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=L)
    log(f"topk row boundary L={L}")
    gc = GpuCache(wl)
    _check(gc, gen.idx_query(wl), 2048)


def _tie_keys(mode):
    def fn(b, k):
        L = k.shape[0]
        if mode == "zeros":
            return np.zeros_like(k)
        rng = np.random.default_rng(b)
        for s in rng.integers(0, max(1, L - 128), 40):       # 40 rows copied onto ~1% each
            k = gen.plant_ties(k, int(s), rng.integers(0, max(1, L - 128), max(1, L // 100)))
        return k
    return fn


@pytest.mark.parametrize("mode", ["planted", "zeros"])
def test_ties_go_to_lower_positions(mode):
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=6000)
    log(f"topk ties mode={mode}")
    gc = GpuCache(wl, keys_fn=_tie_keys(mode))
    q = gen.idx_query(wl)
    for K in (1, 100, 777, 2048):
        _check(gc, q, K)


@pytest.mark.parametrize("mode", ["planted", "zeros"])
def test_ties_past_the_lds_candidate_list(mode):
    """~20K candidates per sequence: with all scores equal every candidate is
    kept, more than the selections hold on chip, so the rest go through
    their global overflow areas."""
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=20000)
    log(f"topk ties L=20000 mode={mode}")
    gc = GpuCache(wl, keys_fn=_tie_keys(mode))
    q = gen.idx_query(wl)
    for K in (2048, 7000, 19000):
        _check(gc, q, K)


def test_multi_block_plan_and_large_K():
    """150K candidates: longer than the one-block selection takes, so the
    filter + final plan runs; K = 65536 overflows its on-chip list too."""
    wl = gen.WORKLOADS["tiny"].with_(L=150_000, Di=64)
    log("topk L=150000 (multi-block plan)")
    gc = GpuCache(wl, keep_kv=False)
    q = gen.idx_query(wl)
    for K in (2048, 65536):
        _check(gc, q, K)


def test_paged_ragged_batch_di128():
    wl = gen.WORKLOADS["b128_rag"].with_(B=16, L=20000, L_min=1, D=128, H=16)
    log("topk paged ragged B=16")
    gc = GpuCache(wl)
    _check(gc, gen.idx_query(wl), 512)


def _clustered_keys(q, block_starts):
    """Keys of 60% of the positions in the given 1024-position blocks made
    small perturbations of the sequence's best key for its query q[b]: those
    blocks then hold far more than their share of the Top-K, with distinct
    scores spread over several top digits."""
    def fn(b, k):
        n = max(0, k.shape[0] - 128)
        best = int(np.argmax(k[:n].astype(np.int64) @ q[b].astype(np.int64)))
        rng = np.random.default_rng(100 + b)
        out = k.copy()
        for s0 in block_starts:
            rows = np.arange(s0, min(s0 + 1024, n))
            rows = rows[rng.random(rows.size) < 0.6]
            noise = rng.integers(-3, 4, size=(rows.size, k.shape[1]))
            out[rows] = np.clip(k[best].astype(np.int64) + noise, -127, 127).astype(np.int8)
        return out
    return fn


def test_clustered_top_scores():
    """Top scores packed into two 1024-position blocks, with distinct scores
    over several top digits: the threshold digit and its ties come from a
    few places, the rest of the sequence far below them."""
    wl = gen.WORKLOADS["tiny"].with_(B=4, L=40000)
    log("topk clustered L=40000")
    q = gen.idx_query(wl)
    gc = GpuCache(wl, keys_fn=_clustered_keys(q, [5 * 1024, 17 * 1024]))
    for K in (300, 1000, 2048):
        _check(gc, q, K)


def test_final_gather_plans():
    """300K candidates (73 filter chunks): with spread-out top scores every
    chunk's kept list fits its group of 8 gathering threads (the direct
    gather); with the top scores packed into two 1024-position blocks, or a
    K that keeps hundreds per chunk, a chunk overflows its group and the
    slot-by-slot search over the chunk offsets runs instead."""
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=300_000, Di=64)
    q = gen.idx_query(wl)
    log("topk L=300000 spread")
    gc = GpuCache(wl, keep_kv=False)
    for K in (2048, 9000):
        _check(gc, q, K)
    del gc
    log("topk L=300000 clustered")
    gc = GpuCache(wl, keep_kv=False, keys_fn=_clustered_keys(q, [40 * 1024, 200 * 1024]))
    _check(gc, q, 2048)


@pytest.mark.parametrize("Di", [64, 128])
def test_many_block_scoring_grid(Di):
    """40 sequences of up to 110K positions: at least 4096 scoring blocks of
    16 pages, so the scoring launch runs 8-page blocks."""
    wl = gen.WORKLOADS["b128_rag"].with_(B=40, L=110_000, L_min=100_000, D=128, H=16, Di=Di)
    log(f"topk many-block scoring grid Di={Di}")
    gc = GpuCache(wl, keep_kv=False)
    _check(gc, gen.idx_query(wl), 2048)


def test_deterministic_and_workspace_reuse():
    """Same call twice on one workspace (the first leaves its control words
    zero) and on a fresh one: identical bits; a shorter max_ctx bound too."""
    wl = gen.WORKLOADS["tiny"].with_(B=3, L=9000)
    gc = GpuCache(wl)
    q = gen.idx_query(wl)
    ws = csa2.Workspace(DEV)
    a = _run(gc, q, 300, ws=ws)
    b = _run(gc, q, 300, ws=ws)
    c = _run(gc, q, 300)
    for x, y in ((a, b), (a, c)):
        assert all(np.array_equal(u, v) for u, v in zip(x, y))
    _check(gc, q, 300, ws=ws)


def test_workspace_shared_across_batch_sizes():
    """One Workspace object for calls of different batch sizes: batch 1 on
    the multi-block plan (150K candidates), then batch 2 with a smaller
    max_ctx, then batch 1 again.  The control words of the batch-2 call sit
    where the batch-1 call's chunk counts and scores were, so the binding
    zeroes the buffer again when the batch changes; every call bit-exact."""
    big = gen.WORKLOADS["tiny"].with_(L=150_000, Di=64)
    small = gen.WORKLOADS["tiny"].with_(B=2, L=9000, Di=64)
    log("topk workspace shared: B=1 L=150000, B=2 L=9000, B=1 again")
    g1, g2 = GpuCache(big, keep_kv=False), GpuCache(small, keep_kv=False)
    ws = csa2.Workspace(DEV)
    for gc in (g1, g2, g1, g2):
        _check(gc, gen.idx_query(gc.wl), 2048, ws=ws)
