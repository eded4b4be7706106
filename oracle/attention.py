"""Sparse attention over the selected global rows merged with the window (oracle).

The global cache and the window cache are merged before decoding
(infernews "DeepSeek V4.1 Flash ... 技術規格剖析", section 2: the window
state of the last 128 tokens is merged with the projected global cache), and
each layer keeps its own 128-token window (zulogic "DeepSeek V4 1-Flash
架构拆解", section 4).  Readings used here, where the pages are silent:

* one latent row per token serves as both key and value;
* the merge is one softmax over the union of the selected positions and the
  window positions [max(0, L-128), L) (no sink, no gate) -- which equals an
  LSE-merge of the two parts computed separately;
* selected rows are the exact dequantised FP4 values, window rows the bf16
  ring values, logits l = sigma * <q_h, x>, o_h = sum softmax(l) x, and
  lse_h = max l + ln sum exp(l - max l) (natural log).
"""
from __future__ import annotations

import numpy as np

from . import formats

WINDOW = 128


def window_positions(L: int) -> np.ndarray:
    return np.arange(max(0, L - WINDOW), L)


def attend(q: np.ndarray, sigma: float, x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Softmax attention of queries q [H, D] over rows x [n, D] (keys = values).

    Returns o [H, D] and lse [H] in float64; for n == 0, o = 0 and lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    H = q.shape[0]
    if x.shape[0] == 0:
        return np.zeros((H, q.shape[1])), np.full(H, -np.inf)
    logits = float(sigma) * (q @ x.T)                    # [H, n]
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    z = w.sum(axis=1, keepdims=True)
    o = (w @ x) / z
    lse = (m + np.log(z))[:, 0]
    return o, lse


def decode_rows(codes: np.ndarray, scales: np.ndarray, ring: np.ndarray,
                sel: np.ndarray, L: int) -> np.ndarray:
    """The rows one query attends to: dequantised FP4 rows of the selected
    positions (in the given order) followed by the window rows of positions
    [max(0, L-128), L) read from ring slot p % 128."""
    glob = formats.dequantize_rows(codes, scales) if len(sel) else np.zeros((0, ring.shape[1]))
    wpos = window_positions(L)
    win = formats.bf16_value(ring[wpos % WINDOW])
    return np.concatenate([glob, win], axis=0)


def sparse_decode(q_bits: np.ndarray, sigma: float, codes: np.ndarray, scales: np.ndarray,
                  ring: np.ndarray, sel: np.ndarray, L: int) -> tuple[np.ndarray, np.ndarray]:
    """One query (all heads) of one sequence: q_bits bf16 [H, D]; (codes,
    scales) the stored rows of the selected positions ``sel``; ring the
    layer's window ring [128, D] bf16."""
    x = decode_rows(codes, scales, ring, sel, L)
    return attend(formats.bf16_value(q_bits), sigma, x)


def dense_reference(q_bits: np.ndarray, sigma: float, x: np.ndarray):
    """Independent dense path for self-checks: torch's scaled-dot-product
    attention on CPU float64 tensors with scale = sigma, over rows x [n, D]."""
    import torch
    q = torch.from_numpy(formats.bf16_value(q_bits))[None, :, None, :]   # [1, H, 1, D]
    k = torch.from_numpy(np.asarray(x, dtype=np.float64))[None, None]    # [1, 1, n, D]
    k = k.expand(1, q.shape[1], -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, k, scale=float(sigma))
    return o[0, :, 0, :].numpy()


def lse_merge(outs, lses) -> tuple[np.ndarray, np.ndarray]:
    """Merge attention results over disjoint key sets (one per shard): with
    M = max_s lse_s, w_s = exp(lse_s - M), the result is
    o = sum_s w_s o_s / sum_s w_s and lse = M + ln sum_s w_s.  A part with no
    keys (lse = -inf) has weight 0; if every part is empty, o = 0 and
    lse = -inf.  Exact in real arithmetic: o_s = sum_j e^(l_j) x_j / e^(lse_s)."""
    outs = [np.asarray(o, dtype=np.float64) for o in outs]
    lses = np.stack([np.asarray(l, dtype=np.float64) for l in lses])      # [n, H]
    M = lses.max(axis=0)
    safe = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - safe), 0.0)             # [n, H]
    z = w.sum(axis=0)
    o = sum(w[s][:, None] * outs[s] for s in range(len(outs)))
    o = np.where(z[:, None] > 0, o / np.where(z > 0, z, 1.0)[:, None], 0.0)
    lse = np.where(z > 0, safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    return o, lse

