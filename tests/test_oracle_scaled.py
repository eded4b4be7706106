"""Pins for the oracle's ranking of scaled indexer scores (a float32 key
scale per token): brute force with Python floats and sorted() on tiny inputs,
the reduction to the integer ranking when every scale is 1, ties between
different (scale, score) pairs, signed zeros, and the single rounding of the
product."""
import numpy as np
import pytest

from oracle import select as S


def _brute(scores, scales, L, K):
    vals = [float(np.float32(np.float32(s) * np.float32(c))) for s, c in zip(scales, scores)]
    vals = [0.0 if v == 0 else v for v in vals]
    cand = list(range(max(0, L - 128)))
    chosen = sorted(sorted(cand, key=lambda p: (-vals[p], p))[:K])
    return chosen + [-1] * (K - len(chosen)), len(chosen)


@pytest.mark.parametrize("seed", range(6))
def test_scaled_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(129, 400))
    scores = rng.integers(-50, 50, L)
    scales = rng.choice(np.array([0.5, 1.0, 1.5, 2.0, -1.0, 3.0, 0.0], np.float32), L)
    v = S.scaled_values(scores, scales)
    for K in (1, 7, 64, 300):
        idx, c, vals = S.topk_values(v, L, K)
        want, wc = _brute(scores, scales, L, K)
        assert c == wc and list(idx) == want
        assert np.array_equal(vals[:c], v[idx[:c]])


def test_unit_scales_reduce_to_integer_ranking():
    rng = np.random.default_rng(7)
    L = 3000
    scores = rng.integers(-2 ** 20, 2 ** 20, L)
    v = S.scaled_values(scores, np.ones(L, np.float32))
    for K in (1, 100, 2900):
        a = S.topk_values(v, L, K)
        b = S.topk(scores, L, K)
        assert a[1] == b[1] and np.array_equal(a[0], b[0])


def test_cross_pair_ties_and_signed_zero():
    # v = 6 from (2, 3) and (3, 2) and (1.5, 4): a three-way tie, lower positions first
    scores = np.array([3, 2, 4, 0, 0, 5] + [0] * 128)
    scales = np.array([2, 3, 1.5, -1, 1, 1] + [1] * 128, np.float32)
    v = S.scaled_values(scores, scales)
    assert not np.signbit(v[3])                         # -1 * 0 counts as +0
    idx, c, _ = S.topk_values(v, len(scores), 3)
    # ranking: 6 (0, 1, 2) then 5 (5) -> top 3 = positions 0, 1, 2
    assert list(idx) == [0, 1, 2]
    idx, c, _ = S.topk_values(v, len(scores), 5)
    assert list(idx) == [0, 1, 2, 3, 5]                 # the two zeros tie: position 3 first

def test_product_rounds_once_to_float32():
    # 2^21 - 1 and a scale with a long mantissa: the product needs rounding
    s = np.float32(1.0 + 2.0 ** -20)
    score = 2 ** 21 - 1
    v = S.scaled_values(np.array([score]), np.array([s]))[0]
    exact = (1.0 + 2.0 ** -20) * score                  # exact in float64
    assert v == np.float32(exact) and float(v) != exact


# ---------------------------------------------------------------- Reindex by values
def _fl32_product(scale, score):
    """fl32(s * score): the float32 x float32 product is exact in a Python
    float (at most 48 significant bits); one rounding to float32 follows."""
    v = float(np.float32(float(np.float32(scale)) * float(score)))
    return 0.0 if v == 0 else v


def _brute_reindex(pool, count, vals_by_pos, K):
    entries = [int(p) for p in pool[:count]]
    ranked = sorted(entries, key=lambda p: (-vals_by_pos[p], p))
    chosen = sorted(ranked[:K])
    return chosen + [-1] * (K - len(chosen)), len(chosen)


_SCALE_SETS = {
    "signed_zero": np.array([0.5, 1.0, -1.0, 0.0, 2.0, -0.25, 3.0], np.float32),
    "fine": (1.0 + np.arange(64) * 2.0 ** -23).astype(np.float32),
    "lognormal": None,
}


@pytest.mark.parametrize("kind", sorted(_SCALE_SETS))
@pytest.mark.parametrize("seed", range(4))
def test_reindex_values_brute_force(kind, seed):
    """A pool built by one indexer query, ranked by the values of another:
    random pools (ascending, and the same set shuffled, with junk past the
    count), signed / zero / last-bit scales, every K edge."""
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(300, 900))
    n = L - 128
    keys = rng.integers(-127, 128, (L, 16)).astype(np.int8)
    q_own, q_pool = (rng.integers(-127, 128, 16).astype(np.int8) for _ in range(2))
    scores = S.indexer_scores(q_own, keys)
    if kind == "fine":
        scores[:] = scores[0]                              # one score, scales differ in the last bits
    if _SCALE_SETS[kind] is None:
        scales = np.exp(rng.standard_normal(L)).astype(np.float32) / np.float32(128)
    else:
        scales = rng.choice(_SCALE_SETS[kind], L)
    v = S.scaled_values(scores, scales)
    vals_by_pos = [_fl32_product(scales[p], int(scores[p])) for p in range(L)]
    assert [float(x) for x in v] == vals_by_pos
    P = int(rng.integers(1, n))
    pool_sc = S.indexer_scores(q_pool, keys[:n])
    pool, count = S.topk(pool_sc, L, P)                   # ascending, -1 padded
    count_used = int(rng.integers(0, count + 1))
    shuffled = pool.copy()
    shuffled[:count_used] = rng.permutation(pool[:count_used])
    shuffled[count_used:] = rng.integers(0, n, P - count_used)   # past the count: ignored
    for pl in (pool, shuffled):
        vop = v[np.maximum(pl, 0)]
        for K in sorted({0, 1, 2, count_used // 2, max(count_used - 1, 0), count_used,
                         count_used + 3}):
            idx, c = S.reindex_values(pl, count_used, vop, K)
            want, wc = _brute_reindex(pl, count_used, vals_by_pos, K)
            assert c == wc and list(idx) == want, (kind, seed, K)


def test_reindex_values_ties_go_to_lower_position_not_pool_slot():
    """Equal values: the lower position wins even when it sits later in the
    pool (a ranking by pool slot would pick 40 here)."""
    pool = np.array([40, 7, 300, 12], np.int32)
    vop = np.array([2.0, 2.0, 5.0, 1.0], np.float32)
    idx, c = S.reindex_values(pool, 4, vop, 2)
    assert c == 2 and list(idx) == [7, 300]
    idx, c = S.reindex_values(pool, 4, vop, 3)
    assert list(idx) == [7, 40, 300]


def test_reindex_values_pool_of_all_candidates_equals_topk_values():
    rng = np.random.default_rng(11)
    L = 2500
    scores = rng.integers(-3000, 3000, L)
    scales = rng.choice(np.array([0.5, 1.0, 2.0, -1.0, 0.0], np.float32), L)
    v = S.scaled_values(scores, scales)
    pool = np.arange(L - 128)
    for K in (1, 77, 1000, L - 128, L):
        a = S.reindex_values(pool, pool.size, v[pool], K)
        b = S.topk_values(v, L, K)
        assert a[1] == b[1] and np.array_equal(a[0], b[0])


def test_reindex_values_prefix_property():
    """Refiltering TopK_P by the same values gives TopK_K' of those values."""
    rng = np.random.default_rng(12)
    L = 4000
    scores = rng.integers(-500, 500, L)
    scales = (2.0 ** rng.integers(-3, 4, L)).astype(np.float32)    # many exact ties
    v = S.scaled_values(scores, scales)
    pool, pc, _ = S.topk_values(v, L, 1500)
    for K2 in (1, 100, 1499, 1500):
        a = S.reindex_values(pool, pc, v[pool[:pc]], K2)
        b = S.topk_values(v, L, K2)
        assert a[1] == b[1] and np.array_equal(a[0][:a[1]], b[0][:b[1]])
