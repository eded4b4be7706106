"""Seeded synthetic inputs for the CSA2 sparse-decode path.

This module draws random numbers and stores them in the input formats the
path consumes (bf16 bit patterns, int8, int32).  It holds none of the
method's arithmetic: no quantisation, no scoring, no selection, no attention.
Both the CPU oracle and the HIP path take their inputs from here, and nothing
here imports either of them.

Every tensor comes from its own NumPy PCG64 stream, keyed by
``SeedSequence([seed, workload_id, tensor_id, layer, b])``, so one sequence
of a large batch can be regenerated on its own without drawing the others.

Workloads (shapes from the benchmark definition of this decode step):

=========  ====  =========================  ==  ===  ==  ==================
name       B     context                    H   D    Di  K
=========  ====  =========================  ==  ===  ==  ==================
tiny       1     4096                       16  128  64  256
b8_64k     8     65536                      64  512  128 2048
chain_64k  8     65536                      64  512  128 Full 8192 -> 2048
b1_1m      1     1048576                    64  512  128 2048 (+3 sigma boost)
b128_rag   128   U{8192..131072}, paged     64  512  128 2048 (+append)
=========  ====  =========================  ==  ===  ==  ==================
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

WINDOW = 128          # sliding-window length, tokens
PAGE = 64             # KV rows per page

# tensor ids for the sub-streams
T_KV, T_KEYS, T_QIDX, T_Q, T_BOOST, T_LENS, T_PERM, T_APPEND_X, T_APPEND_K, T_SWA = range(10)
T_KSCALE = 10


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int                  # workload id, part of every stream key
    B: int
    L: int                    # context length (upper bound when ragged)
    H: int
    D: int
    Di: int
    K: int                    # Top-K of the Full layer
    K2: int = 0               # Top-K' of the Reindex layer (chain only)
    layers: int = 1           # 1 = single Full layer, 3 = Full -> Reindex -> Reuse
    ragged: bool = False      # per-sequence lengths U{L_min..L}
    L_min: int = 0
    paged: bool = False       # globally permuted page table
    boost: float = 0.0        # fraction of positions boosted in indexer space
    append_steps: int = 0     # spare page capacity for appended tokens
    seed: int = 0
    q_std: float | None = None     # std of the query before bf16 rounding
    sigma_mult: float = 1.0        # softmax scale = sigma_mult / sqrt(D)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, B=1, L=4096, H=16, D=128, Di=64, K=256),
    "b8_64k": Workload("b8_64k", 2, B=8, L=65536, H=64, D=512, Di=128, K=2048),
    "chain_64k": Workload("chain_64k", 3, B=8, L=65536, H=64, D=512, Di=128,
                          K=8192, K2=2048, layers=3),
    "b1_1m": Workload("b1_1m", 4, B=1, L=1 << 20, H=64, D=512, Di=128, K=2048,
                      boost=0.01),
    "b128_rag": Workload("b128_rag", 5, B=128, L=131072, L_min=8192, H=64, D=512,
                         Di=128, K=2048, ragged=True, paged=True, append_steps=4),
}


def _rng(wl: Workload, tensor_id: int, layer: int = 0, b: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([wl.seed, wl.wid, tensor_id, layer, b])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); returns uint16 bits.

    Storage conversion of a finite draw into the bf16 input format."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- lengths/pages
def ctx_lens(wl: Workload) -> np.ndarray:
    """Context length L_b of each sequence (int32 [B])."""
    if not wl.ragged:
        return np.full(wl.B, wl.L, dtype=np.int32)
    r = _rng(wl, T_LENS)
    return r.integers(wl.L_min, wl.L, size=wl.B, endpoint=True).astype(np.int32)


def max_pages_per_seq(wl: Workload) -> int:
    return max(1, -(-(wl.L + wl.append_steps) // PAGE))


def page_table(wl: Workload, lens: np.ndarray | None = None) -> tuple[np.ndarray, int]:
    """Logical->physical page map (int32 [B, max_pages]) and the number of
    physical pages.  Contiguous workloads use the identity layout
    (sequence b owns pages [b*mp, (b+1)*mp)); paged workloads scatter every
    sequence's pages through one global random permutation.  Unused entries
    are -1."""
    mp = max_pages_per_seq(wl)
    if lens is None:
        lens = ctx_lens(wl)
    if not wl.paged:
        pt = np.arange(wl.B * mp, dtype=np.int32).reshape(wl.B, mp)
        return pt, wl.B * mp
    need = -(-(lens.astype(np.int64) + wl.append_steps) // PAGE)
    total = max(1, int(need.sum()))      # a cache holds at least one page
    perm = _rng(wl, T_PERM).permutation(total).astype(np.int32)
    pt = np.full((wl.B, mp), -1, dtype=np.int32)
    off = 0
    for b in range(wl.B):
        n = int(need[b])
        pt[b, :n] = perm[off:off + n]
        off += n
    return pt, total


# ---------------------------------------------------------------- tensors
def kv_bf16(wl: Workload, b: int, n: int) -> np.ndarray:
    """Rows [0, n) of sequence b's latent KV tokens, bf16(N(0,1)), uint16 [n, D]."""
    x = _rng(wl, T_KV, 0, b).standard_normal(n * wl.D, dtype=np.float32)
    return f32_to_bf16_bits(x).reshape(n, wl.D)


def idx_query(wl: Workload, layer: int = 0) -> np.ndarray:
    """One int8 indexer query vector per sequence, U{-127..127}: int8 [B, Di]."""
    r = _rng(wl, T_QIDX, layer)
    return r.integers(-127, 127, size=(wl.B, wl.Di), endpoint=True, dtype=np.int8)


def idx_keys(wl: Workload, b: int, n: int) -> np.ndarray:
    """Indexer keys of sequence b, int8 [n, Di], U{-127..127}.

    With ``wl.boost`` > 0 a Bernoulli(boost) subset of positions is pushed
    towards the layer-0 indexer query by three key standard deviations:
    k <- clip(k + rint(3 * sd_k * q / ||q||_2), -127, 127), sd_k the std of
    U{-127..127}.  This makes the Top-K set non-trivial at long context."""
    k = _rng(wl, T_KEYS, 0, b).integers(-127, 127, size=(n, wl.Di), endpoint=True,
                                         dtype=np.int8)
    if wl.boost > 0:
        q = idx_query(wl, 0)[b].astype(np.float64)
        sd_k = math.sqrt((255.0 ** 2 - 1.0) / 12.0)
        delta = np.rint(3.0 * sd_k * q / np.linalg.norm(q)).astype(np.int32)
        mask = _rng(wl, T_BOOST, 0, b).random(n) < wl.boost
        kb = k[mask].astype(np.int32) + delta[None, :]
        k[mask] = np.clip(kb, -127, 127).astype(np.int8)
    return k


def key_scales(wl: Workload, b: int, n: int, mode: str = "lognormal") -> np.ndarray:
    """Per-token fp32 indexer-key scales of sequence b, float32 [n].

    lognormal  exp(N(0, 1)) / 128: positive, spread over about two decades
               (the magnitude of an absmax / 127 quantisation scale)
    pow2       2^U{-3..3}: products of different scores collide exactly
    fine       1 + U{0..1023} * 2^-23: equal scores give values that differ
               only in their lowest mantissa bits
    signed     lognormal with a random sign, and about 5% exact zeros
    subnormal  lognormal times 2^-140: most products are float32 subnormals"""
    r = _rng(wl, T_KSCALE, 0, b)
    if mode == "pow2":
        return np.ldexp(np.float32(1.0), r.integers(-3, 3, size=n, endpoint=True)).astype(np.float32)
    if mode == "fine":
        return (np.float32(1.0) + r.integers(0, 1023, size=n, endpoint=True).astype(np.float32)
                * np.float32(2.0 ** -23)).astype(np.float32)
    s = (np.exp(r.standard_normal(n)) / 128.0).astype(np.float32)
    if mode == "signed":
        s = np.where(r.random(n) < 0.5, -s, s).astype(np.float32)
        s[r.random(n) < 0.05] = np.float32(0.0)
    elif mode == "subnormal":
        s = (s * np.float32(2.0 ** -140)).astype(np.float32)
    elif mode != "lognormal":
        raise ValueError(f"unknown key-scale mode {mode!r}")
    return s


def key_scales_e4m3(wl: Workload, b: int, n: int) -> np.ndarray:
    """Per-token indexer-key scales as E4M3 bytes, uint8 [n]: codes
    U{0x00..0x7E} (every finite non-negative value, zero included)."""
    return _rng(wl, T_KSCALE, 1, b).integers(0, 0x7E, size=n, endpoint=True).astype(np.uint8)


def query(wl: Workload, layer: int = 0) -> np.ndarray:
    """Attention queries, bf16(N(0,1) * std) with std = 1/sqrt(D) by default:
    uint16 [B, H, D]."""
    std = wl.q_std if wl.q_std is not None else 1.0 / math.sqrt(wl.D)
    x = _rng(wl, T_Q, layer).standard_normal(wl.B * wl.H * wl.D, dtype=np.float32)
    return f32_to_bf16_bits(x * np.float32(std)).reshape(wl.B, wl.H, wl.D)


def softmax_scale(wl: Workload) -> np.float32:
    return np.float32(wl.sigma_mult / math.sqrt(wl.D))


def swa_ring(wl: Workload, kv: np.ndarray, L: int) -> np.ndarray:
    """Sliding-window ring of one sequence: the bf16 tokens at positions
    [max(0, L-W), L), each in slot pos % W; other slots zero.  uint16 [W, D]."""
    ring = np.zeros((WINDOW, wl.D), dtype=np.uint16)
    lo = max(0, L - WINDOW)
    pos = np.arange(lo, L)
    ring[pos % WINDOW] = kv[lo:L]
    return ring


def layer_ring(wl: Workload, b: int, L: int, layer: int, kv_tail: np.ndarray | None = None) -> np.ndarray:
    """Window ring of layer ``layer`` for sequence b at length L (uint16 [W, D]).

    Layer 0 (the cache owner) windows the same tokens that were quantised
    into the FP4 cache: pass their bf16 rows [max(0, L-W), L) as ``kv_tail``.
    Every other layer keeps its own window state; its tokens are an
    independent bf16(N(0,1)) draw."""
    lo = max(0, L - WINDOW)
    if layer == 0:
        assert kv_tail is not None and kv_tail.shape[0] == L - lo
        rows = kv_tail
    else:
        x = _rng(wl, T_SWA, layer, b).standard_normal((L - lo) * wl.D, dtype=np.float32)
        rows = f32_to_bf16_bits(x).reshape(L - lo, wl.D)
    ring = np.zeros((WINDOW, wl.D), dtype=np.uint16)
    ring[np.arange(lo, L) % WINDOW] = rows
    return ring


def append_tokens(wl: Workload, step: int) -> tuple[np.ndarray, np.ndarray]:
    """One new token per sequence for decode step ``step``:
    bf16(N(0,1)) uint16 [B, D] and int8 keys [B, Di]."""
    xs = np.empty((wl.B, wl.D), dtype=np.uint16)
    ks = np.empty((wl.B, wl.Di), dtype=np.int8)
    for b in range(wl.B):
        xs[b] = f32_to_bf16_bits(
            _rng(wl, T_APPEND_X, step, b).standard_normal(wl.D, dtype=np.float32))
        ks[b] = _rng(wl, T_APPEND_K, step, b).integers(-127, 127, size=wl.Di,
                                                         endpoint=True, dtype=np.int8)
    return xs, ks


# ---------------------------------------------------------------- test variants
def plant_ties(keys: np.ndarray, src: int, dst: np.ndarray) -> np.ndarray:
    """Copy the key row at ``src`` onto the rows ``dst`` so that those
    positions score exactly alike under any query (ties planted on purpose)."""
    out = keys.copy()
    out[dst] = keys[src]
    return out
