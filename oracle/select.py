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


# ---------------------------------------------------------------- sharding
# Context sharding of one long sequence (one shard per device, contiguous page
# ranges): each shard ranks its own candidates under the same total order and
# keeps its local Top-K; the global Top-K is then the Top-K of the union of the
# local lists.  This holds because the order is total: an entry of the global
# Top-K is beaten by fewer than K entries overall, hence by fewer than K in its
# own shard, so it is in that shard's local list.  (The pages do not describe
# sharding; this is the reading of the method's selection rule applied to a
# partition of the candidates.)

def topk_range(scores: np.ndarray, L: int, K: int, p_begin: int,
               p_end: int) -> tuple[np.ndarray, int, np.ndarray]:
    """Shard-local selection over candidates p_begin <= p < min(p_end, L-128),
    ranked as in ``topk``.  Returns (positions ascending, padded with -1 to K;
    count; the scores of those positions, 0 past the count)."""
    hi = min(p_end, max(0, L - WINDOW))
    pos = np.arange(p_begin, hi) if hi > p_begin else np.zeros(0, dtype=np.int64)
    order = rank_order(scores[pos], pos)
    idx, c = _emit(pos[order[:min(K, pos.size)]], K)
    sc = np.zeros(K, dtype=np.int64)
    sc[:c] = np.asarray(scores)[idx[:c]]
    return idx, c, sc


def merge_topk(parts, K: int) -> tuple[np.ndarray, int]:
    """Global selection from shard-local lists over disjoint position sets:
    ``parts`` holds (positions, count, scores) per shard; the union is ranked
    by (score desc, position asc), the first min(K, total) kept, emitted
    ascending and padded with -1."""
    pos = np.concatenate([np.asarray(p[0][:p[1]], dtype=np.int64) for p in parts])
    sc = np.concatenate([np.asarray(p[2][:p[1]], dtype=np.int64) for p in parts])
    order = rank_order(sc, pos)
    return _emit(pos[order[:min(K, pos.size)]], K)


# ---------------------------------------------------------------- key scales
# Indexer keys with a scale per token (the pages name the indexer "K / scale"
# but give no formula).  Reading: each cached position p carries an fp32
# scale s_p; the ranked value is v_p = fl32(s_p * score_p), the product
# rounded once to float32 (round to nearest, ties to even); ranking is by v
# descending, then position ascending, with -0 and +0 equal (a tie); scales
# must be finite.  The integer score is exact in float32 (|score| <= 2^21).

def scaled_values(scores: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """v = fl32(s * score) for int scores and float32 scales; -0 becomes +0."""
    v = np.asarray(scales, dtype=np.float32) * np.asarray(scores, dtype=np.int64).astype(np.float32)
    v = v.astype(np.float32)
    v[v == 0] = np.float32(0.0)
    return v


def rank_order_values(values: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Permutation sorting entries by (value descending, position ascending)."""
    v = np.asarray(values, dtype=np.float64)          # exact widening of float32
    return np.lexsort((np.asarray(pos), -v))


def topk_values(values: np.ndarray, L: int, K: int) -> tuple[np.ndarray, int, np.ndarray]:
    """Full-layer selection ranked by float values over candidates [0, L-128):
    (positions ascending, -1 padded to K; count; their values, 0 past it)."""
    n = max(0, L - WINDOW)
    pos = np.arange(n)
    order = rank_order_values(values[:n], pos)
    idx, c = _emit(pos[order[:min(K, n)]], K)
    vals = np.zeros(K, dtype=np.float32)
    vals[:c] = np.asarray(values, dtype=np.float32)[idx[:c]]
    return idx, c, vals


def reindex_values(pool: np.ndarray, pool_count: int, values_of_pool: np.ndarray,
                   K: int) -> tuple[np.ndarray, int]:
    """Reindex layer ranked by float values of the pool entries."""
    p = np.asarray(pool[:pool_count], dtype=np.int64)
    order = rank_order_values(values_of_pool[:pool_count], p)
    return _emit(p[order[:min(K, pool_count)]], K)

