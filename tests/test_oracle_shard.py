"""Pins for the oracle's context-sharded selection and LSE merge.

The merged shard-local Top-K must equal the one-device Top-K (pinned itself by
brute force in test_oracle_select.py) for random partitions, planted ties,
empty shards and K beyond the candidates; the LSE merge of attention over a
partition of the keys must equal attention over all keys (the plain softmax
definition)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import select as S


def _shards(L, n, rng, page=64):
    """n page-aligned, ascending, disjoint ranges covering [0, L)."""
    pages = -(-L // page)
    cuts = np.sort(rng.choice(np.arange(1, max(2, pages)), size=min(n - 1, max(0, pages - 1)),
                              replace=False)) if pages > 1 else np.zeros(0, dtype=int)
    bounds = [0] + [int(c) * page for c in cuts] + [L]
    return list(zip(bounds[:-1], bounds[1:]))


@pytest.mark.parametrize("seed", range(12))
def test_merged_shard_topk_equals_one_device(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(130, 5000))
    scores = rng.integers(-40, 40, L).astype(np.int64)     # narrow range: many ties
    if seed % 3 == 0:
        scores[:] = 7                                      # all equal
    for K in (1, 17, 256, 5000):
        n = int(rng.integers(1, 9))
        parts = [S.topk_range(scores, L, K, a, b) for a, b in _shards(L, n, rng)]
        got = S.merge_topk(parts, K)
        want = S.topk(scores, L, K)
        assert got[1] == want[1] and np.array_equal(got[0], want[0]), (seed, K, n)


def test_range_topk_scores_and_empty_shards():
    rng = np.random.default_rng(99)
    L = 1000
    scores = rng.integers(-1000, 1000, L).astype(np.int64)
    idx, c, sc = S.topk_range(scores, L, 10, 64, 320)
    assert c == 10 and np.all((idx[:c] >= 64) & (idx[:c] < 320))
    assert np.array_equal(sc[:c], scores[idx[:c]]) and np.all(sc[c:] == 0)
    # a shard wholly inside the window and one past the end hold no candidates
    for a, b in ((L - 128, L), (2000, 3000)):
        idx, c, sc = S.topk_range(scores, L, 10, a, b)
        assert c == 0 and np.all(idx == -1)
    got = S.merge_topk([S.topk_range(scores, L, 10, L - 128, L)], 10)
    assert got[1] == 0 and np.all(got[0] == -1)


@pytest.mark.parametrize("n", [1, 2, 5])
def test_lse_merge_equals_attention_over_all_keys(n):
    rng = np.random.default_rng(n)
    H, D, m = 4, 32, 300
    q = rng.normal(size=(H, D))
    x = rng.normal(size=(m, D)) * 3.0
    sigma = 0.7
    o, lse = A.attend(q, sigma, x)
    cuts = np.sort(rng.choice(np.arange(1, m), size=n - 1, replace=False))
    parts = [A.attend(q, sigma, x[a:b]) for a, b in zip([0, *cuts], [*cuts, m])]
    o2, lse2 = A.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    assert np.max(np.abs(o2 - o)) < 1e-12 and np.max(np.abs(lse2 - lse)) < 1e-12


def test_lse_merge_empty_parts():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(2, 8))
    x = rng.normal(size=(5, 8))
    o, lse = A.attend(q, 0.5, x)
    e = A.attend(q, 0.5, x[:0])                            # no keys: o = 0, lse = -inf
    o2, lse2 = A.lse_merge([e[0], o, e[0]], [e[1], lse, e[1]])
    assert np.max(np.abs(o2 - o)) < 1e-14 and np.max(np.abs(lse2 - lse)) < 1e-14
    o3, lse3 = A.lse_merge([e[0], e[0]], [e[1], e[1]])
    assert np.all(o3 == 0) and np.all(np.isneginf(lse3))
