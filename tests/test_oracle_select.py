"""Pins for the oracle's indexer scores, Top-K, Reindex and Reuse.

Brute force in Python integers and Python's sorted() on tiny inputs (every
K, planted ties), an O(L) separation invariant at larger sizes, and the
special cases that reduce Reindex to Top-K."""
import numpy as np
import pytest

from harness import gen
from oracle import select as S


def _brute_scores(q, keys):
    return [sum(int(a) * int(b) for a, b in zip(q, row)) for row in keys]


def _brute_topk(scores, L, K):
    cand = list(range(max(0, L - 128)))
    ranked = sorted(cand, key=lambda p: (-scores[p], p))
    chosen = sorted(ranked[:K])
    return chosen + [-1] * (K - len(chosen)), len(chosen)


@pytest.mark.parametrize("Di", [16, 64, 128])
def test_scores_brute_force(Di):
    rng = np.random.default_rng(Di)
    q = rng.integers(-127, 128, Di).astype(np.int8)
    k = rng.integers(-127, 128, (50, Di)).astype(np.int8)
    assert list(S.indexer_scores(q, k)) == _brute_scores(q, k)


def test_scores_extreme_bound():
    q = np.full(128, -127, dtype=np.int8)
    k = np.full((2, 128), 127, dtype=np.int8)
    k[1] = -127
    s = S.indexer_scores(q, k)
    assert list(s) == [-127 * 127 * 128, 127 * 127 * 128]
    assert abs(int(s[0])) < 2 ** 31


@pytest.mark.parametrize("L", [0, 1, 127, 128, 129, 200, 300])
def test_topk_brute_force_all_K(L):
    rng = np.random.default_rng(L)
    # small value range -> many ties at every threshold
    scores = rng.integers(-3, 4, max(L, 1)).astype(np.int64)
    for K in range(0, max(0, L - 128) + 3):
        got, cnt = S.topk(scores, L, K)
        want, wcnt = _brute_topk(list(scores), L, K)
        assert cnt == wcnt and list(got) == want, (L, K)


def test_topk_planted_ties_take_lower_positions():
    scores = np.zeros(1000, dtype=np.int64)
    scores[[10, 500, 700, 871]] = 5                # four tied top scores
    idx, cnt = S.topk(scores, 1000, 2)
    assert cnt == 2 and list(idx) == [10, 500]
    idx, cnt = S.topk(scores, 1000, 6)             # then the lowest-position zeros
    assert list(idx) == [0, 1, 10, 500, 700, 871]


def test_topk_separation_invariant_large():
    rng = np.random.default_rng(7)
    L, K = 70000, 2048
    scores = rng.integers(-2_000_000, 2_000_001, L).astype(np.int64)
    scores[rng.integers(0, L, 5000)] = scores[123]  # ties around one value
    idx, cnt = S.topk(scores, L, K)
    sel = idx[:cnt]
    assert cnt == K and np.all(np.diff(sel) > 0) and np.all(idx[cnt:] == -1)
    mask = np.zeros(L - 128, bool)
    mask[sel] = True
    key_sel = np.stack([scores[:L - 128][mask], -np.nonzero(mask)[0]], 1)
    key_uns = np.stack([scores[:L - 128][~mask], -np.nonzero(~mask)[0]], 1)
    worst_sel = min(map(tuple, key_sel))
    best_uns = max(map(tuple, key_uns))
    assert worst_sel > best_uns


def test_reindex_pool_all_candidates_equals_topk():
    rng = np.random.default_rng(3)
    L = 2000
    keys = rng.integers(-127, 128, (L, 64)).astype(np.int8)
    q = rng.integers(-127, 128, 64).astype(np.int8)
    sc = S.indexer_scores(q, keys)
    pool = np.arange(L - 128)
    for K in (1, 100, 1872, 2000):
        a = S.reindex(pool, pool.size, sc[pool], K)
        b = S.topk(sc, L, K)
        assert a[1] == b[1] and np.array_equal(a[0], b[0])


def test_reindex_prefix_property():
    """Refiltering TopK_P(q0) with the same query q0 gives TopK_K'(q0)."""
    rng = np.random.default_rng(4)
    L = 5000
    keys = rng.integers(-127, 128, (L, 64)).astype(np.int8)
    keys = gen.plant_ties(keys, 17, np.arange(100, 4000, 37))
    q = rng.integers(-127, 128, 64).astype(np.int8)
    sc = S.indexer_scores(q, keys)
    pool, pc = S.topk(sc, L, 1024)
    for K2 in (1, 256, 1000, 1024):
        a = S.reindex(pool, pc, sc[pool[:pc]], K2)
        b = S.topk(sc, L, K2)
        assert a[1] == b[1] and np.array_equal(a[0][:a[1]], b[0][:b[1]])
    a = S.reindex(pool, pc, sc[pool[:pc]], 1500)     # K' beyond the pool keeps it all
    assert a[1] == pc and np.array_equal(a[0][:pc], pool[:pc]) and np.all(a[0][pc:] == -1)


def test_reuse_is_identity():
    idx = np.array([3, 9, -1], dtype=np.int32)
    out, c = S.reuse(idx, 2)
    assert c == 2 and np.array_equal(out, idx) and out is not idx


def test_reindex_brute_force_shuffled_pools():
    """Integer Reindex against Python sorted(): a pool chosen by one query,
    ranked by another; ascending and shuffled pools, junk past the count."""
    rng = np.random.default_rng(21)
    for trial in range(6):
        L = int(rng.integers(200, 700))
        n = L - 128
        keys = rng.integers(-4, 5, (L, 8)).astype(np.int8)        # small range: many ties
        q_own, q_pool = (rng.integers(-127, 128, 8).astype(np.int8) for _ in range(2))
        sc = S.indexer_scores(q_own, keys)
        brute = _brute_scores(q_own, keys)
        pool, count = S.topk(S.indexer_scores(q_pool, keys[:n]), L, int(rng.integers(1, n)))
        shuffled = pool.copy()
        shuffled[:count] = rng.permutation(pool[:count])
        shuffled[count:] = rng.integers(0, n, pool.size - count)
        for pl in (pool, shuffled):
            for K in (0, 1, count // 3, count, count + 5):
                got, c = S.reindex(pl, count, sc[np.maximum(pl, 0)], K)
                ranked = sorted((int(p) for p in pl[:count]), key=lambda p: (-brute[p], p))
                want = sorted(ranked[:K])
                assert c == len(want) and list(got) == want + [-1] * (K - len(want))
