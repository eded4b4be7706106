"""Pins for the oracle's merged sparse attention.

K = all candidates reduces to dense attention, checked against torch's
scaled_dot_product_attention in float64 (a library routine); closed forms
(q = 0 gives the mean, one key gives that key); the joint softmax equals an
LSE merge of the selected part and the window part; order invariance."""
import math

import numpy as np
import pytest

from harness import gen
from oracle import attention as A
from oracle import formats as F
from oracle import select as S


def _tiny(L=600, D=128, H=16, seed=0, q_std=None):
    wl = gen.WORKLOADS["tiny"].with_(L=L, seed=seed, q_std=q_std)
    kv = gen.kv_bf16(wl, 0, L)
    ring = gen.swa_ring(wl, kv, L)
    q = gen.query(wl, 0)[0]
    return wl, kv, ring, q


@pytest.mark.parametrize("q_std", [None, 1.0])
def test_all_selected_equals_dense_sdpa(q_std):
    wl, kv, ring, q = _tiny(q_std=q_std)
    L = wl.L
    n = L - 128
    sel = np.arange(n)
    codes, scales = F.quantize_rows(kv[:n])
    sigma = float(gen.softmax_scale(wl))
    o, lse = A.sparse_decode(q, sigma, codes, scales, ring, sel, L)
    x = np.concatenate([F.dequantize_rows(codes, scales), F.bf16_value(kv[n:L])])
    ref = A.dense_reference(q, sigma, x)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_zero_query_gives_mean():
    wl, kv, ring, q = _tiny()
    sel = np.array([5, 40, 77])
    codes, scales = F.quantize_rows(kv[sel])
    o, lse = A.sparse_decode(np.zeros_like(q), 0.1, codes, scales, ring, sel, wl.L)
    x = A.decode_rows(codes, scales, ring, sel, wl.L)
    assert np.allclose(o, x.mean(0)[None, :], atol=1e-14, rtol=0)
    assert np.allclose(lse, math.log(len(x)))


def test_single_key_returns_it():
    q = gen.f32_to_bf16_bits(np.linspace(-1, 1, 4 * 64, dtype=np.float32)).reshape(4, 64)
    x = np.linspace(-3, 3, 64)[None, :]
    o, lse = A.attend(F.bf16_value(q), 0.125, x)
    assert np.array_equal(o, np.repeat(x, 4, 0))
    assert np.allclose(lse, 0.125 * F.bf16_value(q) @ x[0])


def test_lse_merge_of_parts_equals_joint():
    wl, kv, ring, q = _tiny()
    sel = np.arange(0, 400, 3)
    codes, scales = F.quantize_rows(kv[sel])
    sigma = 0.2
    qf = F.bf16_value(q)
    xg = F.dequantize_rows(codes, scales)
    xw = F.bf16_value(ring[A.window_positions(wl.L) % 128])
    o1, l1 = A.attend(qf, sigma, xg)
    o2, l2 = A.attend(qf, sigma, xw)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    om = (w1[:, None] * o1 + w2[:, None] * o2) / (w1 + w2)[:, None]
    o, lse = A.sparse_decode(q, sigma, codes, scales, ring, sel, wl.L)
    assert np.max(np.abs(o - om)) < 1e-13
    assert np.max(np.abs(lse - (m + np.log(w1 + w2)))) < 1e-12


def test_order_invariance():
    wl, kv, ring, q = _tiny()
    sel = np.arange(10, 450, 7)
    perm = np.random.default_rng(0).permutation(sel.size)
    c1, s1 = F.quantize_rows(kv[sel])
    o1, _ = A.sparse_decode(q, 0.3, c1, s1, ring, sel, wl.L)
    o2, _ = A.sparse_decode(q, 0.3, c1[perm], s1[perm], ring, sel[perm], wl.L)
    assert np.max(np.abs(o1 - o2)) < 1e-13


def test_short_context_window_only():
    """L < 128: no global candidates, the window covers [0, L)."""
    wl, kv, ring, q = _tiny(L=50)
    idx, cnt = S.topk(np.zeros(50, np.int64), 50, 16)
    assert cnt == 0
    o, lse = A.sparse_decode(q, 0.1, np.zeros((0, 64), np.uint8), np.zeros((0, 8), np.uint8),
                             ring, idx[:0], 50)
    ref = A.dense_reference(q, 0.1, F.bf16_value(kv[:50]))
    assert np.max(np.abs(o - ref)) < 1e-12


def test_empty_context():
    o, lse = A.attend(np.ones((2, 8)), 1.0, np.zeros((0, 8)))
    assert np.all(o == 0) and np.all(np.isneginf(lse))
