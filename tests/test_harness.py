"""The seeded input generators: determinism, per-sequence sub-streams,
shapes and value ranges."""
import numpy as np

from harness import gen


def test_deterministic_and_substreams():
    wl = gen.WORKLOADS["b8_64k"]
    a = gen.kv_bf16(wl, 3, 100)
    b = gen.kv_bf16(wl, 3, 100)
    c = gen.kv_bf16(wl, 4, 100)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert np.array_equal(gen.kv_bf16(wl, 3, 50), a[:50])
    assert gen.query(wl).shape == (8, 64, 512)
    q = gen.idx_query(wl)
    assert q.dtype == np.int8 and q.min() >= -127 and q.shape == (8, 128)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], np.float32)
    assert list(gen.f32_to_bf16_bits(x)) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


def test_ragged_paged_layout():
    wl = gen.WORKLOADS["b128_rag"]
    lens = gen.ctx_lens(wl)
    assert lens.min() >= 8192 and lens.max() <= 131072
    pt, total = gen.page_table(wl, lens)
    used = pt[pt >= 0]
    assert used.size == total and np.array_equal(np.sort(used), np.arange(total))
    need = -(-(lens + wl.append_steps) // 64)
    assert np.all((pt >= 0).sum(1) == need)


def test_boost_moves_keys_towards_query():
    wl = gen.WORKLOADS["b1_1m"]
    k = gen.idx_keys(wl, 0, 20000).astype(np.int64)
    k0 = gen.idx_keys(wl.with_(boost=0.0), 0, 20000).astype(np.int64)
    q = gen.idx_query(wl, 0)[0].astype(np.int64)
    moved = np.any(k != k0, axis=1)
    assert 100 < moved.sum() < 300
    assert np.all((k[moved] @ q) > (k0[moved] @ q))
