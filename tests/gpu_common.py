"""Shared set-up of the GPU parity tests.

Builds a CSA2 cache on the GPU from the seeded harness draws (through
csa2_quantize_append), keeps the host draws the oracle needs, and provides
oracle-side references computed from those same host draws only.
"""
from __future__ import annotations

import contextlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import fp4_compressed_sparse_csa2_amd as csa2
from harness import gen
from oracle import attention as OA
from oracle import formats as OF
from oracle import select as OS

DEV = torch.device("cuda:0")
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
ATOL = 2e-3          # max-abs bound on attention outputs against the fp64 oracle


def log(msg: str) -> None:
    print(msg, flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


class GpuCache:
    """A cache filled on the GPU with sequence b's tokens at positions [0, L_b)."""

    def __init__(self, wl: gen.Workload, layers: int = 1, keep_kv: bool = True, keys_fn=None):
        self.wl = wl
        self.lens = gen.ctx_lens(wl)
        self.pt, self.npages = gen.page_table(wl, self.lens)
        self.cache = csa2.Cache.allocate(wl.B, self.pt.shape[1], self.npages, wl.D, wl.Di,
                                         torch.from_numpy(self.pt), DEV)
        self.kv = [None] * wl.B
        self.keys = [None] * wl.B
        rings = np.zeros((layers, wl.B, gen.WINDOW, wl.D), dtype=np.uint16)

        def draw(b):
            L = int(self.lens[b])
            keys = gen.idx_keys(wl, b, L)
            if keys_fn is not None:
                keys = keys_fn(b, keys)
            return b, gen.kv_bf16(wl, b, L), keys

        with ThreadPoolExecutor(THREADS) as ex:
            for b, kv, keys in ex.map(draw, range(wl.B)):
                L = int(self.lens[b])
                if L > 0:
                    csa2.quantize_append(self.cache, to_dev(kv),
                                         torch.full((L,), b, dtype=torch.int32, device=DEV),
                                         torch.arange(L, dtype=torch.int32, device=DEV),
                                         keys=to_dev(keys))
                lo = max(0, L - gen.WINDOW)
                for layer in range(layers):
                    rings[layer, b] = gen.layer_ring(wl, b, L, layer, kv[lo:L])
                self.keys[b] = keys
                if keep_kv:
                    self.kv[b] = kv
        self.swa = [to_dev(rings[i]) for i in range(layers)]
        self.rings = rings
        self.ctx = to_dev(self.lens.astype(np.int32))
        torch.cuda.synchronize()

    def kv_rows(self, b: int, pos: np.ndarray) -> np.ndarray:
        """Host bf16 rows of sequence b at positions ``pos`` (regenerated if not kept)."""
        kv = self.kv[b]
        if kv is None:
            kv = gen.kv_bf16(self.wl, b, int(self.lens[b]))
        return kv[pos]


# ------------------------------------------------------------------ oracle side
def oracle_topk(keys: np.ndarray, q_idx: np.ndarray, L: int, K: int):
    sc = OS.indexer_scores(q_idx, keys[:max(0, L - gen.WINDOW)])
    idx, cnt = OS.topk(sc, L, K)
    return sc, idx, cnt


def oracle_decode(q_bits: np.ndarray, sigma: float, kv_sel: np.ndarray, ring: np.ndarray,
                  sel: np.ndarray, L: int):
    """Oracle attention of one sequence: selected rows are quantised by the
    oracle from their bf16 draws (never read back from the GPU)."""
    if len(sel):
        codes, scales = OF.quantize_rows(kv_sel)
    else:
        codes = np.zeros((0, q_bits.shape[1] // 2), np.uint8)
        scales = np.zeros((0, q_bits.shape[1] // 16), np.uint8)
    return OA.sparse_decode(q_bits, sigma, codes, scales, ring, sel, L)


def assert_close(got: np.ndarray, want: np.ndarray, atol: float, what: str) -> float:
    err = float(np.max(np.abs(got.astype(np.float64) - want))) if got.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= atol, f"{what}: max-abs error {err:.3e} > {atol:.1e}"
    return err


# Decode plans a test can force through the library's tuning variables:
# (heads per block, FP4 tiles per split or None for the library's choice).
DECODE_PLANS = {
    "auto": (None, None),
    "hg64": ("64", None),
    "hg64_split3": ("64", "3"),
    "hg64_split1": ("64", "1"),
    "hg16_split2": ("16", "2"),
    "hg16_split4": ("16", "4"),
    "hg64_split5": ("64", "5"),
}


@contextlib.contextmanager
def decode_plan(name: str):
    """Run csa2_sparse_decode calls under the named plan (environment
    variables read by the library on every call), then restore."""
    hg, tps = DECODE_PLANS[name]
    keys = {"CSA2_DECODE_HEADS_PER_BLOCK": hg, "CSA2_DECODE_SPLIT_TILES": tps}
    old = {k: os.environ.get(k) for k in keys}
    try:
        for k, v in keys.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
