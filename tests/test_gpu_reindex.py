"""GPU parity of csa2_reindex: the Reindex layer's scores and Top-K' over the
Full layer's pool, bit-exact against the oracle (pool smaller than K',
K' = P, pools from short contexts padded with -1, planted ties, pool lengths
around the one-block selection's load rows and past its limit)."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen
from oracle import cache as OC
from oracle import select as OS

from gpu_common import DEV, GpuCache, log, oracle_topk, to_dev, to_host

pytestmark = pytest.mark.gpu


def _chain(gc: GpuCache, K_full: int, K2: int):
    wl = gc.wl
    q0, q1 = gen.idx_query(wl, 0), gen.idx_query(wl, 1)
    max_ctx = max(1, int(gc.lens.max()))
    pool, pc = csa2.index_topk(gc.cache, gc.ctx, max_ctx, to_dev(q0), K_full, csa2.Workspace(DEV))
    sc = torch.full((wl.B, K_full), -7, dtype=torch.int32, device=DEV)
    idx, cnt = csa2.reindex(gc.cache, to_dev(q1), pool, pc, K2, csa2.Workspace(DEV), out_scores=sc)
    torch.cuda.synchronize()
    pool_h, pc_h, idx_h, cnt_h, sc_h = map(to_host, (pool, pc, idx, cnt, sc))
    for b in range(wl.B):
        L = int(gc.lens[b])
        _, wpool, wpc = oracle_topk(gc.keys[b], q0[b], L, K_full)
        assert int(pc_h[b]) == wpc and np.array_equal(pool_h[b], wpool), f"pool b={b}"
        p = wpool[:wpc]
        s2 = OS.indexer_scores(q1[b], gc.keys[b][p])
        want, wcnt = OS.reindex(wpool, wpc, s2, K2)
        if wpc > K2:                                  # scores are produced when a selection runs
            assert np.array_equal(sc_h[b, :wpc], s2), f"reindex scores b={b}"
        assert int(cnt_h[b]) == wcnt and np.array_equal(idx_h[b], want), f"reindex idx b={b}"


@pytest.mark.parametrize("K_full,K2", [(1024, 256), (1024, 1024), (512, 1), (3000, 2000)])
def test_chain_small(K_full, K2):
    wl = gen.WORKLOADS["tiny"].with_(B=3, L=6000, Di=128)
    log(f"reindex K_full={K_full} K2={K2}")
    _chain(GpuCache(wl), K_full, K2)


@pytest.mark.parametrize("K_full,K2", [(1023, 300), (4097, 1000), (4099, 4098), (12290, 3000),
                                       (16383, 2048), (16384, 5000), (20000, 2048)])
def test_chain_pool_sizes(K_full, K2):
    """Pools whose length is not a multiple of 4 (read entry by entry), that
    cross the one-block selection's 4096-entry load rows, fill all four, or
    exceed them (the filter plan mapping pool entries)."""
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=21000, Di=128)
    log(f"reindex pool sizes K_full={K_full} K2={K2}")
    _chain(GpuCache(wl), K_full, K2)


def test_page_table_past_lds_stage():
    """A 70K-token context (1094 pages): the scoring kernel reads the page
    table from global memory instead of its 1024-entry LDS copy."""
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=70_000, Di=64)
    log("reindex 70K context (page table past the LDS stage)")
    _chain(GpuCache(wl, keep_kv=False), 3000, 1000)


def test_short_pools():
    """Contexts of 0..900 tokens: pools shorter than K', padded with -1."""
    wl = gen.WORKLOADS["b128_rag"].with_(B=12, L=900, L_min=0, D=128, H=16, Di=64)
    log("reindex short pools")
    _chain(GpuCache(wl), 512, 200)


def test_reindex_ties():
    def fn(b, k):
        rng = np.random.default_rng(10 + b)
        for s in rng.integers(0, 4000, 30):
            k = gen.plant_ties(k, int(s), rng.integers(0, 4000, 80))
        return k
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=4300, Di=64)
    log("reindex planted ties")
    _chain(GpuCache(wl, keys_fn=fn), 2048, 300)
