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
