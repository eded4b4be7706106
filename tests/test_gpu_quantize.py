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
