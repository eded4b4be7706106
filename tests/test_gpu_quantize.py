"""GPU parity of csa2_quantize_append against the oracle: page bytes (E2M1
codes, E4M3 scales, indexer keys) bit-exact, window-ring slots bit-exact.

The codec sweep drives every non-negative finite E4M3 scale code through the
kernel (group maximum 6*s) and, for each, every finite bf16 value that can sit
in such a group, in both signs."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen
from oracle import cache as OC
from oracle import formats as OF

from gpu_common import DEV, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _sweep_rows(D: int) -> np.ndarray:
    """bf16 rows whose 16-channel groups cover every scale code and, per code,
    every finite bf16 magnitude <= 6*s (both signs, -0 included)."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    allb = allb[((allb >> 7) & 0xFF) != 0xFF]
    vals = OF.bf16_value(allb)
    groups = []
    for sc in range(127):
        amax = 6.0 * OF.e4m3_value(sc)
        abits = gen.f32_to_bf16_bits(np.array([amax], np.float32))[0]
        assert OF.bf16_value(abits) == amax
        members = allb[np.abs(vals) <= amax]
        n_g = -(-members.size // 15)
        pad = np.resize(members, n_g * 15).reshape(n_g, 15)
        g = np.empty((n_g, 16), np.uint16)
        for i in range(n_g):                      # amax at a rotating channel
            j = i % 16
            g[i, :j], g[i, j], g[i, j + 1:] = pad[i, :j], abits, pad[i, j:]
        groups.append(g)
    groups = np.concatenate(groups)
    per_row = D // 16
    n_rows = -(-groups.shape[0] // per_row)
    groups = np.resize(groups, (n_rows * per_row, 16))
    return groups.reshape(n_rows, D)


def _extra_rows(D: int) -> np.ndarray:
    rng = np.random.default_rng(5)
    rows = [gen.f32_to_bf16_bits(rng.standard_normal((64, D)).astype(np.float32)),
            gen.f32_to_bf16_bits((rng.standard_normal((16, D)) * 1e30).astype(np.float32)),
            gen.f32_to_bf16_bits((rng.standard_normal((16, D)) * 1e-30).astype(np.float32)),
            np.zeros((2, D), np.uint16), np.full((2, D), 0x8000, np.uint16)]
    return np.concatenate(rows)


@pytest.mark.parametrize("D,Di", [(512, 128), (128, 64), (256, 64)])
def test_codec_sweep_bit_exact(D, Di):
    x = np.concatenate([_sweep_rows(D), _extra_rows(D)])
    n = x.shape[0]
    log(f"quantize sweep D={D} Di={Di}: {n} rows")
    mp = -(-n // 64)
    pt = np.arange(mp, dtype=np.int32)[None, :]
    cache = csa2.Cache.allocate(1, mp, mp, D, Di, torch.from_numpy(pt), DEV)
    keys = np.random.default_rng(1).integers(-127, 128, (n, Di)).astype(np.int8)
    csa2.quantize_append(cache, to_dev(x), torch.zeros(n, dtype=torch.int32, device=DEV),
                         torch.arange(n, dtype=torch.int32, device=DEV), keys=to_dev(keys))
    got = to_host(cache.pages)
    want = np.zeros_like(got)
    OC.append(want, pt, D, Di, np.zeros(n, int), np.arange(n), x, keys, None)
    # rows beyond n in the last page were never written on either side
    assert np.array_equal(got, want)


def _every_amax_rows(D: int) -> np.ndarray:
    """One 16-channel group per finite non-negative bf16 value as its group
    maximum (all 32,640 of them, +0 included): the maximum sits at a rotating
    channel, the other 15 channels are random bf16 values of magnitude at most
    the maximum, both signs, a third of them at an E2M1 midpoint times amax/6
    (next to the element rounding boundaries).  So the scale rounding of amax/6 is driven through the
    kernel for every amax it can see, not only at the centre of each scale
    code's interval."""
    allb = np.arange(1 << 15, dtype=np.uint32).astype(np.uint16)        # sign bit clear
    allb = allb[((allb >> 7) & 0xFF) != 0xFF]                           # finite: 32,640 values
    assert allb.size == 32640
    amax = OF.bf16_value(allb)
    rng = np.random.default_rng(32640)
    u = rng.uniform(-1.0, 1.0, (allb.size, 15))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])            # E2M1 midpoints / 6
    tie = rng.random((allb.size, 15)) < 1.0 / 3.0
    u = np.where(tie, rng.choice(mids, (allb.size, 15)) * np.sign(u) / 6.0, u)
    vals = (u * amax[:, None]).astype(np.float32)
    bits = gen.f32_to_bf16_bits(vals)
    over = np.abs(OF.bf16_value(bits)) > amax[:, None]                   # rounded past the max
    bits = np.where(over, allb[:, None] | (bits & np.uint16(0x8000)), bits)
    g = np.empty((allb.size, 16), np.uint16)
    for j in range(16):
        sel = np.arange(allb.size) % 16 == j
        g[sel, :j], g[sel, j], g[sel, j + 1:] = bits[sel, :j], allb[sel], bits[sel, j:]
    assert np.all(np.max(np.abs(OF.bf16_value(g)), axis=1) == amax)
    per_row = D // 16
    n_rows = -(-g.shape[0] // per_row)
    return np.resize(g, (n_rows * per_row, 16)).reshape(n_rows, D)


@pytest.mark.parametrize("D,Di", [(512, 128), (128, 64)])
def test_every_bf16_amax_bit_exact(D, Di):
    x = _every_amax_rows(D)
    n = x.shape[0]
    log(f"quantize every-amax D={D}: {n} rows, 32640 groups")
    mp = -(-n // 64)
    pt = np.arange(mp, dtype=np.int32)[None, :]
    cache = csa2.Cache.allocate(1, mp, mp, D, Di, torch.from_numpy(pt), DEV)
    csa2.quantize_append(cache, to_dev(x), torch.zeros(n, dtype=torch.int32, device=DEV),
                         torch.arange(n, dtype=torch.int32, device=DEV))
    got = to_host(cache.pages)
    want = np.zeros_like(got)
    OC.append(want, pt, D, Di, np.zeros(n, int), np.arange(n), x, None, None)
    assert np.array_equal(got, want)


def test_window_ring_and_paged_append():
    wl = gen.WORKLOADS["tiny"].with_(B=3, L=500, paged=True, append_steps=0)
    lens = np.array([500, 130, 70], np.int32)
    pt, npages = gen.page_table(wl, lens)
    D, Di = wl.D, wl.Di
    cache = csa2.Cache.allocate(3, pt.shape[1], npages, D, Di, torch.from_numpy(pt), DEV)
    swa = torch.zeros((3, 128, D), dtype=torch.uint16, device=DEV)
    want_pages = np.zeros((npages, OC.page_bytes(D, Di)), np.uint8)
    want_swa = np.zeros((3, 128, D), np.uint16)
    for b in range(3):
        L = int(lens[b])
        kv = gen.kv_bf16(wl, b, L)
        keys = gen.idx_keys(wl, b, L)
        # bulk fill without the window, then the last <=128 tokens with it
        lo = max(0, L - 128)
        csa2.quantize_append(cache, to_dev(kv[:lo]), torch.full((lo,), b, dtype=torch.int32, device=DEV),
                             torch.arange(lo, dtype=torch.int32, device=DEV), keys=to_dev(keys[:lo]))
        csa2.quantize_append(cache, to_dev(kv[lo:]), torch.full((L - lo,), b, dtype=torch.int32, device=DEV),
                             torch.arange(lo, L, dtype=torch.int32, device=DEV), keys=to_dev(keys[lo:]),
                             swa=swa)
        OC.append(want_pages, pt, D, Di, np.full(L, b), np.arange(L), kv, keys, None)
        OC.append(want_pages, pt, D, Di, np.full(L - lo, b), np.arange(lo, L), kv[lo:], keys[lo:],
                  want_swa)
    assert np.array_equal(to_host(cache.pages), want_pages)
    assert np.array_equal(to_host(swa), want_swa)


def test_out_of_range_tokens_are_skipped():
    D, Di = 128, 64
    pt = np.array([[0, 1]], np.int32)
    cache = csa2.Cache.allocate(1, 2, 2, D, Di, torch.from_numpy(pt), DEV)
    x = gen.f32_to_bf16_bits(np.ones((4, D), np.float32))
    seq = np.array([0, 1, -1, 0], np.int32)       # b = 1 and b = -1 do not exist
    pos = np.array([5, 5, 5, 128], np.int32)      # 128 is beyond 2 pages
    csa2.quantize_append(cache, to_dev(x), to_dev(seq), to_dev(pos))
    got = to_host(cache.pages)
    want = np.zeros_like(got)
    OC.append(want, pt, D, Di, np.array([0]), np.array([5]), x[:1], None, None)
    assert np.array_equal(got, want)
