"""Indexer scoring, deterministic Top-K, Reindex and Reuse (oracle).

The pages: every attention layer is statically one of Full, Reindex or Reuse;
layers share the main KV and the indexer keys, and the Top-K addressing
indices are reused across layers; a later indexer layer only refilters the
candidate pool that the first Full layer built (neodrop V4.1-Flash report,
"架构拆解" item 2; zulogic "DeepSeek V4 1-Flash 架构拆解", section 3 mode
table).  The pages give no scoring formula; the readings used here:

* score(p) = sum_d q[d] * k[p, d] over int8 query and keys, an exact integer
  (no activation, no per-head weights, no key scale);
* candidates of a Full layer are the positions outside the sliding window,
  0 <= p < L - 128;
* ranking is by score descending, then position ascending (ties go to the
  lower position);
* the selected positions are returned in ascending order, padded with -1 to
  K, together with their count min(K, #candidates).
"""
from __future__ import annotations

import numpy as np

WINDOW = 128


def indexer_scores(q_idx: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """score[p] = sum_d q[d]*k[p,d]  (int8 x int8 -> int64), exact.

    The product runs in float64, which is exact here: every partial sum is
    bounded by 127*127*Di < 2**53."""
    q = np.asarray(q_idx, dtype=np.int8).astype(np.float64)
    k = np.asarray(keys, dtype=np.int8).astype(np.float64)
    return (k @ q).astype(np.int64)


def rank_order(scores: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Permutation sorting entries by (score descending, position ascending)."""
    return np.lexsort((np.asarray(pos), -np.asarray(scores, dtype=np.int64)))


def _emit(chosen: np.ndarray, K: int) -> tuple[np.ndarray, int]:
    out = np.full(K, -1, dtype=np.int32)
    chosen = np.sort(np.asarray(chosen, dtype=np.int64))
    out[:chosen.size] = chosen
    return out, int(chosen.size)


def topk(scores: np.ndarray, L: int, K: int) -> tuple[np.ndarray, int]:
    """Full-layer selection over candidates [0, L-128): the first min(K, n) in
    (score desc, position asc) order, emitted ascending and padded with -1.

    ``scores`` covers at least the candidate positions."""
    n = max(0, L - WINDOW)
    pos = np.arange(n)
    order = rank_order(scores[:n], pos)
    return _emit(pos[order[:min(K, n)]], K)


def reindex(pool: np.ndarray, pool_count: int, scores_of_pool: np.ndarray,
            K: int) -> tuple[np.ndarray, int]:
    """Reindex layer: rank the first ``pool_count`` pool entries (a set of
    positions) by this layer's own scores, keep the first min(K, count),
    emit ascending, pad with -1.  ``scores_of_pool[i]`` scores pool[i]."""
    p = np.asarray(pool[:pool_count], dtype=np.int64)
    order = rank_order(scores_of_pool[:pool_count], p)
    return _emit(p[order[:min(K, pool_count)]], K)


def reuse(idx: np.ndarray, count: int) -> tuple[np.ndarray, int]:
    """Reuse layer: the owner's (or the Reindex layer's) selection, unchanged."""
    return np.array(idx, copy=True), int(count)
