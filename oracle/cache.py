"""The compressed global cache and the per-layer window ring (oracle).

One owner ("Full") layer holds the compressed global KV, the indexer keys and
the selection metadata, and consumer layers read them through aliases
(zulogic "DeepSeek V4 1-Flash 架构拆解", section 3, owner/consumer diagram);
every layer also keeps its own 128-token sliding-window state with a shorter
lifetime (same page, section 4; infernews "DeepSeek V4.1 Flash ...
技術規格剖析", section 2).

Byte layout (the library's documented cache format, restated here on its
own): the cache is an array of pages of 64 token positions.  A page is

    rows   [64][R]     R = D/2 + D/16 bytes per token:
                         codes  [D/2]   E2M1 codes, channel 2j low nibble of byte j
                         scales [D/16]  E4M3 scale of channels 16g..16g+15 in byte g
    keys   [64][Di]    int8 indexer keys

back to back, so a page takes 64*(D/2 + D/16 + Di) bytes.  Position p of
sequence b lives in physical page ``page_table[b][p // 64]``, row p % 64.
The window ring of a layer is bf16 [B][128][D], slot = position % 128.
"""
from __future__ import annotations

import numpy as np

from . import formats

PAGE = 64
WINDOW = 128


def page_bytes(D: int, Di: int) -> int:
    return PAGE * (D // 2 + D // 16 + Di)


def _row_bytes(D: int) -> int:
    return D // 2 + D // 16


def _keys_offset(D: int) -> int:
    return PAGE * _row_bytes(D)


def append(pages: np.ndarray, page_table: np.ndarray, D: int, Di: int,
           seq: np.ndarray, pos: np.ndarray, x_bits: np.ndarray,
           keys: np.ndarray | None, swa: np.ndarray | None) -> None:
    """Write tokens into the cache in place (uint8 ``pages`` [num_pages, page_bytes]).

    For each token i: its FP4 row (codes + scales) goes to position pos[i] of
    sequence seq[i]; its indexer key (if given) next to it; its bf16 value to
    window slot pos[i] % 128 of ``swa`` (uint16 [B, 128, D], if given)."""
    codes, scales = formats.quantize_rows(x_bits)
    R, k_off = _row_bytes(D), _keys_offset(D)
    for i in range(len(seq)):
        b, p = int(seq[i]), int(pos[i])
        pg, r = int(page_table[b, p // PAGE]), p % PAGE
        pages[pg, r * R:r * R + D // 2] = codes[i]
        pages[pg, r * R + D // 2:(r + 1) * R] = scales[i]
        if keys is not None:
            pages[pg, k_off + r * Di:k_off + (r + 1) * Di] = keys[i].view(np.uint8)
        if swa is not None:
            swa[b, p % WINDOW] = x_bits[i]


def rows_of(pages: np.ndarray, page_table: np.ndarray, D: int, Di: int,
            b: int, pos: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Stored (codes [n, D/2], scales [n, D/16]) of positions ``pos`` of sequence b."""
    R = _row_bytes(D)
    pos = np.asarray(pos, dtype=np.int64)
    pg = page_table[b, pos // PAGE].astype(np.int64)
    r = pos % PAGE
    ci = r[:, None] * R + np.arange(D // 2)[None, :]
    si = r[:, None] * R + D // 2 + np.arange(D // 16)[None, :]
    return pages[pg[:, None], ci], pages[pg[:, None], si]


def row_byte_index(page_table: np.ndarray, D: int, Di: int, b: int,
                   pos: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Flat byte indices, into the pages array seen as one byte vector, of the
    codes [n, D/2] and scales [n, D/16] of positions ``pos`` of sequence b."""
    R = _row_bytes(D)
    pos = np.asarray(pos, dtype=np.int64)
    base = page_table[b, pos // PAGE].astype(np.int64)[:, None] * page_bytes(D, Di)
    r = (pos % PAGE)[:, None]
    return (base + r * R + np.arange(D // 2)[None, :],
            base + r * R + D // 2 + np.arange(D // 16)[None, :])


def keys_of(pages: np.ndarray, page_table: np.ndarray, D: int, Di: int,
            b: int, pos: np.ndarray) -> np.ndarray:
    """Stored int8 indexer keys [n, Di] of positions ``pos`` of sequence b."""
    k_off = _keys_offset(D)
    pos = np.asarray(pos, dtype=np.int64)
    pg = page_table[b, pos // PAGE].astype(np.int64)
    ki = k_off + ((pos % PAGE)[:, None] * Di + np.arange(Di)[None, :])
    return pages[pg[:, None], ki].view(np.int8)
