"""GPU parity of a multi-layer decode step under a static mode schedule: one
owner cache shared by every layer, Full layers selecting over the context,
Reindex layers refiltering a Full layer's pool with their own indexer query,
Reuse layers aliasing an earlier layer's indices; every layer with its own
queries and window ring.  Indices bit-exact and outputs within the decode
tolerance of the oracle, layer by layer."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from fp4_compressed_sparse_csa2_amd.schedule import FULL, REINDEX, REUSE, Layer, Runner, Schedule
from harness import gen
from oracle import select as OS

from gpu_common import ATOL, DEV, GpuCache, assert_close, log, oracle_decode, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_eight_layer_schedule():
    wl = gen.WORKLOADS["tiny"].with_(B=2, L=9000)
    sched = Schedule([Layer(FULL, 1024), Layer(REINDEX, 256), Layer(REUSE), Layer(REUSE),
                      Layer(REINDEX, 128, source=0), Layer(REUSE), Layer(FULL, 512), Layer(REUSE)])
    n = len(sched.layers)
    log(f"schedule of {n} layers")
    gc = GpuCache(wl, layers=n)
    sigma = float(gen.softmax_scale(wl))
    q_idx_h = {i: gen.idx_query(wl, i) for i in sched.selecting_layers()}
    q_h = [gen.query(wl, i) for i in range(n)]
    outs = [torch.empty((wl.B, wl.H, wl.D), dtype=torch.float32, device=DEV) for _ in range(n)]
    lses = [torch.empty((wl.B, wl.H), dtype=torch.float32, device=DEV) for _ in range(n)]
    run = Runner(sched, gc.cache)
    run.step(gc.ctx, int(gc.lens.max()), {i: to_dev(v) for i, v in q_idx_h.items()},
             [to_dev(v) for v in q_h], gc.swa, sigma, outs, lses)
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(wl.B):
        L = int(gc.lens[b])
        want = {}                                      # the oracle's selection of every layer
        for i, l in enumerate(sched.layers):
            if l.mode == FULL:
                sc = OS.indexer_scores(q_idx_h[i][b], gc.keys[b][:L - gen.WINDOW])
                want[i] = OS.topk(sc, L, l.k)
            elif l.mode == REINDEX:
                pool, pc = want[sched.pool_owner[i]]
                psc = OS.indexer_scores(q_idx_h[i][b], gc.keys[b][pool[:pc]])
                want[i] = OS.reindex(pool, pc, psc, l.k)
            idx, cnt = run.indices(i)
            w_idx, w_cnt = want[sched.index_owner[i]]
            assert int(to_host(cnt)[b]) == w_cnt, f"layer {i} count b={b}"
            assert np.array_equal(to_host(idx)[b], w_idx), f"layer {i} indices b={b}"
            sel = w_idx[:w_cnt]
            o, lz = oracle_decode(q_h[i][b], sigma, gc.kv_rows(b, sel), gc.rings[i, b], sel, L)
            worst = max(worst, assert_close(to_host(outs[i])[b], o, ATOL, f"layer {i} out b={b}"))
            assert_close(to_host(lses[i])[b], lz, ATOL, f"layer {i} lse b={b}")
    # Reuse layers alias their source's tensors
    assert run.indices(2)[0].data_ptr() == run.indices(1)[0].data_ptr()
    assert run.indices(5)[0].data_ptr() == run.indices(4)[0].data_ptr()
    log(f"  {n} layers: indices bit-exact, outputs max-abs error {worst:.2e}")
