"""FP4 E2M1 elements with one E4M3 scale per 16 channels (oracle).

The main KV cache stores every latent channel as a 4-bit E2M1 number and
every group of 16 consecutive channels carries one 8-bit E4M3 scale
(neodrop V4.1-Flash report, "架构拆解" item 3, FP4 main KV cache).  The pages
name the two formats and the group size only; the rest is fixed here:

* E2M1 and E4M3 are read as the OCP definitions: E2M1 = 1 sign, 2 exponent
  bits (bias 1), 1 mantissa bit, exponent field 0 subnormal, no Inf/NaN;
  E4M3 = the "FN" variant, 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
  exponent field 0 subnormal, S.1111.111 = NaN (never produced), max 448.
* Group scale s = E4M3(amax / 6): the group's largest magnitude maps onto the
  largest E2M1 magnitude, 6.  Rounding is to the nearest E4M3 value, ties to
  the even code; anything above 448 saturates to 448.
* Element code: the nearest value in {0, .5, 1, 1.5, 2, 3, 4, 6} * s to |x|,
  ties to the even code; the sign bit is the sign bit of x (so -0 -> 0x8).
  If s = 0 every magnitude code is 0.
* Packing: channel 2j in the low nibble of byte j, channel 2j+1 in the high
  nibble; group g covers channels 16g .. 16g+15.

All comparisons are exact: bf16 inputs, E4M3 values, E2M1 values and their
products have few significant bits and are exact in float64, and the scale
search compares amax against 6*v (exact) instead of amax/6 against v.
"""
from __future__ import annotations

import numpy as np

GROUP = 16


# ------------------------------------------------------------------ decoding
def e2m1_value(code) -> np.ndarray:
    """Value of a 4-bit E2M1 code (sign bit 3, exponent bits 2..1, mantissa bit 0)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64)))
    return sign * mag


def e4m3_value(byte) -> np.ndarray:
    """Value of an E4M3 (FN) byte; NaN for S.1111.111."""
    b = np.asarray(byte, dtype=np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


E2M1_MAG = e2m1_value(np.arange(8))            # 0, .5, 1, 1.5, 2, 3, 4, 6
E4M3_MAG = e4m3_value(np.arange(127))          # codes 0x00..0x7E, ascending, 0..448


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ nearest search
def nearest_even(grid: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Index k minimising |v - grid[..., k]|, ties to the even k.

    ``grid`` has the candidate values on its last axis and broadcasts against
    ``v[..., None]``.  For a strictly increasing grid at most two adjacent
    entries tie, and exactly one of them has an even index; if every entry
    ties (an all-zero grid) the result is 0.  Values beyond the last entry
    land on it (saturation).  Brute force over every candidate."""
    v = np.asarray(v, dtype=np.float64)
    d = np.abs(v[..., None] - grid)
    nearest = d == d.min(axis=-1, keepdims=True)
    even = nearest & (np.arange(grid.shape[-1]) % 2 == 0)
    idx = np.where(even.any(axis=-1), np.argmax(even, axis=-1),
                   np.argmax(nearest, axis=-1)).astype(np.int64)
    # At or beyond the last candidate the nearest one is the last (saturation).
    # Stated outright because, for v many binades above the grid, every float64
    # distance rounds to the same number and the search above would see a tie.
    top = np.broadcast_to(grid[..., -1], idx.shape)
    return np.where((v >= top) & (top > 0), grid.shape[-1] - 1, idx)


def e4m3_scale_code(amax) -> np.ndarray:
    """E4M3 code of s = amax/6: nearest finite non-negative E4M3 value, ties to
    the even code, saturating at 448 (code 0x7E).

    Compares amax against 6*v for every candidate v, which orders and ties
    exactly as amax/6 against v but needs no division (6*v is exact)."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.empty(amax.shape, dtype=np.int64)
    flat, res = amax.reshape(-1), out.reshape(-1)
    for i in range(0, flat.size, 1 << 15):
        res[i:i + (1 << 15)] = nearest_even(6.0 * E4M3_MAG, flat[i:i + (1 << 15)])
    return out


def e2m1_mag_code(xabs, s) -> np.ndarray:
    """E2M1 magnitude code (0..7) of |x| against the grid E2M1 * s, nearest with
    ties to the even code; 0 where s == 0.  ``xabs`` and ``s`` broadcast."""
    xabs, s = np.broadcast_arrays(np.asarray(xabs, dtype=np.float64),
                                  np.asarray(s, dtype=np.float64))
    out = np.empty(xabs.shape, dtype=np.int64)
    fx, fs, res = xabs.reshape(-1), s.reshape(-1), out.reshape(-1)
    for i in range(0, fx.size, 1 << 18):
        sl = slice(i, i + (1 << 18))
        res[sl] = nearest_even(E2M1_MAG[None, :] * fs[sl, None], fx[sl])
    return np.where(s > 0, out, 0)


# ------------------------------------------------------------------ one row
def quantize_rows(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantise bf16 rows [n, D] to (codes uint8 [n, D/2], scales uint8 [n, D/16]).

    Per 16-channel group: amax -> E4M3 scale code -> E2M1 code of every
    channel against that scale's value; two codes per byte, even channel low."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    n, D = x_bits.shape
    assert D % GROUP == 0
    x = bf16_value(x_bits)
    assert np.all(np.isfinite(x)), "non-finite input is outside the contract"
    xg = x.reshape(n, D // GROUP, GROUP)
    amax = np.max(np.abs(xg), axis=2)                           # [n, G]
    sc = e4m3_scale_code(amax)                                  # [n, G]
    s = E4M3_MAG[sc]                                            # [n, G]
    sfull = np.repeat(s, GROUP, axis=1).reshape(n, D)
    mag = e2m1_mag_code(np.abs(x), sfull)
    sign = (x_bits >> np.uint16(15)).astype(np.int64)           # sign bit of x (keeps -0)
    code = (sign << 3) | mag                                    # [n, D]
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc.astype(np.uint8)


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(codes [n, D/2], scales [n, D/16]) -> float64 [n, D]: E2M1(code) * E4M3(scale)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, half = codes.shape
    D = 2 * half
    c = np.empty((n, D), dtype=np.int64)
    c[:, 0::2] = codes & 0xF
    c[:, 1::2] = codes >> 4
    s = e4m3_value(np.asarray(scales, dtype=np.uint8))          # [n, D/16]
    return e2m1_value(c) * np.repeat(s, GROUP, axis=1)
