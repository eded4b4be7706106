"""Pins for the oracle's FP4 codec (E2M1 elements, E4M3 scale per 16 channels).

Each check ties the oracle to something other than itself: a standard's
value table, torch's float8_e4m3fn conversion (a library routine),
hand-worked groups, an independent threshold formulation, or exhaustive
round trips."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F


def _finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 7) & 0xFF) != 0xFF]


def test_e2m1_values_match_ocp_table(golden_dir):
    rows = [l.split() for l in open(os.path.join(golden_dir, "ocp_e2m1.txt"))
            if l.strip() and not l.startswith("#")]
    for code_hex, val in rows:
        code = int(code_hex, 16)
        v = F.e2m1_value(code)
        assert v == float(val) and np.signbit(v) == val.startswith("-"), code_hex


def test_e2m1_invariants():
    mags = F.e2m1_value(np.arange(8))
    assert np.all(np.diff(mags) > 0)
    assert mags.max() == 6.0
    # negative codes mirror positive ones
    assert np.array_equal(F.e2m1_value(np.arange(8) | 8), -mags)


def test_e4m3_decode_matches_torch_all_bytes():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.e4m3_value(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], ours[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_scale_rule_exhaustive_vs_torch():
    """Every non-negative finite bf16 amax: s = E4M3_RNE(amax/6), compared
    with torch's float8_e4m3fn rounding where torch does not saturate, and
    with saturation to 0x7E above that."""
    bits = _finite_bf16()
    bits = bits[bits < 0x8000]                                  # non-negative
    amax = F.bf16_value(bits)
    code = F.e4m3_scale_code(amax)
    q = amax / 6.0
    inrange = q <= 448.0
    t = torch.from_numpy(q[inrange]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(code[inrange], t.astype(np.int64))
    assert np.all(code[~inrange] == 0x7E)
    assert bits.size == 32640


def _mag_code_by_thresholds(xabs, s):
    """Independent formulation: count the midpoints between consecutive E2M1
    magnitudes (taken from the OCP value table) that |x| lies above; a value
    exactly on a midpoint goes to the even neighbour."""
    vals = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    code = np.zeros(np.shape(xabs), dtype=np.int64)
    for k in range(7):
        mid = (vals[k] + vals[k + 1]) / 2.0 * s
        code += (xabs > mid) | ((xabs == mid) & ((k + 1) % 2 == 0))
    return np.where(s > 0, code, 0)


def test_element_code_exhaustive_all_bf16_all_scales():
    """All finite bf16 inputs x all 127 non-negative finite E4M3 scales."""
    x = F.bf16_value(_finite_bf16())
    s_all = F.e4m3_value(np.arange(127))
    xa = np.abs(x)
    for s in s_all:
        ours = F.e2m1_mag_code(xa, s)
        ref = _mag_code_by_thresholds(xa, s)
        assert np.array_equal(ours, ref), s


def test_element_code_round_trip():
    """Every exact grid point E2M1[c]*s encodes back to c (all c, all s > 0)."""
    mags = F.e2m1_value(np.arange(8))
    for s in F.e4m3_value(np.arange(1, 127)):
        assert np.array_equal(F.e2m1_mag_code(mags * s, s), np.arange(8))


def test_element_code_midpoints_go_even():
    mags = F.e2m1_value(np.arange(8))
    for s in (2.0 ** -9, 0.25, 1.0, 1.125, 448.0):
        mids = (mags[:-1] + mags[1:]) / 2 * s
        got = F.e2m1_mag_code(mids, s)
        want = [k if k % 2 == 0 else k + 1 for k in range(7)]
        assert list(got) == want


def test_hand_worked_groups(golden_dir):
    n = 0
    for line in open(os.path.join(golden_dir, "quant_groups.txt")):
        if line.startswith("#") or not line.strip():
            continue
        xs, sc, cs = (p.split() for p in line.split("|"))
        x = np.array([[int(v, 16) for v in xs]], dtype=np.uint16)
        codes, scales = F.quantize_rows(x)
        assert int(scales[0, 0]) == int(sc[0], 16), line
        assert [int(c) for c in codes[0]] == [int(v, 16) for v in cs], line
        n += 1
    assert n == 7


def test_quantize_dequantize_error_bound():
    """Dequantised value is within half a grid step of x (or saturated),
    and the group maximum is never off by more than a quarter scale step."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4096, 128)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)            # truncation: any bf16 will do
    codes, scales = F.quantize_rows(bits)
    y = F.dequantize_rows(codes, scales)
    xv = F.bf16_value(bits)
    s = np.repeat(F.e4m3_value(scales), 16, axis=1)
    # nearest on a grid whose widest gap is 2*s (between 4s and 6s)
    assert np.all(np.abs(y - xv) <= s * 1.0 + 1e-300)
    assert np.all(np.sign(y[y != 0]) == np.sign(xv[y != 0]))


def test_packing_even_channel_low_nibble():
    x = np.zeros((1, 16), dtype=np.uint16)
    x[0, 0] = 0x40C0      # 6.0  -> amax, code 7 on s = 1
    x[0, 1] = 0x3F00      # 0.5  -> code 1
    codes, scales = F.quantize_rows(x)
    assert codes[0, 0] == 0x17 and scales[0, 0] == 0x38


def test_signed_zero_and_negatives():
    x = np.zeros((1, 16), dtype=np.uint16)
    x[0, 0] = 0x3F80      # 1.0
    x[0, 1] = 0x8000      # -0.0
    x[0, 2] = 0xB800      # tiny negative -> magnitude 0, sign kept
    codes, _ = F.quantize_rows(x)
    assert codes[0, 0] >> 4 == 0x8 and codes[0, 1] & 0xF == 0x8
