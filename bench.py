#!/usr/bin/env python3
"""Decode-step benchmark of the CSA2 sparse-decode library on one MI355X.

Workload ``b8_64k``: batch 8, each sequence 65,536 cached tokens; one Full
layer with 64 query heads over one latent KV of width 512 stored as FP4 E2M1
with one E4M3 scale per 16 channels (288 B per token), int8 indexer keys of
width 128, Top-K 2048 over the positions outside the 128-token window, and a
bf16 window ring of 128 tokens.  Inputs are seeded synthetic draws (bf16
N(0,1) latent rows, int8 U{-127..127} keys and indexer query, bf16
N(0,1)/sqrt(512) queries, softmax scale 1/sqrt(512)).

One step = one decode step of every sequence at this layer, all in the
library's HIP kernels, on one stream:

  csa2_quantize_append  the step's new token (position L-1) into the FP4 page,
                        the indexer keys and the window ring
  csa2_index_topk       int8 scores over the 65,408 candidates, Top-2048
  csa2_sparse_decode    64 heads over 2048 FP4 rows + 128 window rows

Re-appending token L-1 rewrites identical bytes, so every step sees the same
cache.  A query is one sequence's new token at this layer (all heads); the
metric is queries per second over the whole job, and the achieved HBM rate
is the algorithmic bytes of a step (what the method must move: keys, the
selected rows, the window, queries, outputs) divided by its time.

Timing.  Inputs are resident in HBM before the timed region.  The caches are
replicated and the steps rotate over the replicas so that no step finds its
keys in the 256 MB last-level cache.  Steps are captured in HIP graphs
(torch.cuda.CUDAGraph) and replayed; the timed region is bracketed by
torch.cuda.synchronize() and HIP events on the stream the kernels run on;
``value``, ``ms_per_step`` and ``hbm_gbs`` all come from those events (the
host wall clock is reported beside them).  A second timed region replays
graphs of one library call at a time to give each call's average duration;
the dominant call (csa2_append_index_topk) is priced against the HBM
roofline, and against the library's read-only stream kernel
(csa2_stream_read over 2 GiB) timed in the same run.

``cpu_baseline`` times the plain CPU oracle (the checker, not the product) on
the same seeded workload: whole decode steps of the 8 sequences, repeated
until about --cpu-seconds of CPU time.  This leg is the only part of the
benchmark that runs the oracle; it also checks the GPU step's eager result
(every sequence: indices bit-exact, outputs within 2e-3) and the scaled
indexer's selection of sequence 0, and fills ``parity`` from them.

Extra legs in the same line (skipped with --no-extras): the three-layer
chain on this cache (Full Top-K 8192 and its decode over the 8192, Reindex
to 2048 and its decode, a Reuse decode; each call and the whole chain step)
and a 20-layer schedule, the scaled indexer, the 128-sequence ragged paged
workload (contexts U{8192..131072}, one appended token per sequence per
step), where the decode call moves enough bytes to be priced against the
HBM roofline on its own (``--ragged-only`` runs that leg alone), and the
one-sequence 1M-token workload's step with its own roofline figure, checked
against the oracle in the CPU leg.

Prints one JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA, vendor figure
WORKLOAD = "b8_64k"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse() -> argparse.Namespace:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=5,
                    help="cache copies the steps rotate over (>= 1 GB in total)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the chain, schedule and scaled-indexer timings (profiling runs: "
                         "only the step's kernels and their per-call timings are launched)")
    ap.add_argument("--ragged-only", action="store_true",
                    help="run only the 128-sequence ragged paged workload and print its JSON")
    ap.add_argument("--counter-run", action="store_true",
                    help="for rocprofv3 --pmc: three 1 GiB device copies (the counter "
                         "calibration), then --warmup + --steps eager steps; no timing")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the FETCH_SIZE and WRITE_SIZE counter runs of --counter-run "
                         "into profiles/traffic.json and exit")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="instead of a run: per-kernel median durations and gaps of each "
                         "workload's step in a rocprofv3 --kernel-trace CSV of this script "
                         "(markdown tables)")
    ap.add_argument("--dcp", type=int, default=0, metavar="N",
                    help="instead of the headline bench: the 1M-token sequence cut over N "
                         "emulated devices (range Top-K per shard, merge, shard decodes, LSE "
                         "merge) against the one-device step, one JSON line")
    return ap.parse_args()


# ------------------------------------------------------------------ byte counts
def algorithmic_bytes(B, L, H, D, Di, K, W=128):
    """Bytes per step each call must move (per query figures times B)."""
    R = D // 2 + D // 16
    n = max(0, L - W)
    topk = n * Di + Di + 4 * K + 4 * (-(-n // 64)) + 4
    decode = K * (R + 4) + W * D * 2 + H * D * 2 + H * D * 4 + 4 * H + 4
    append = (2 * D + Di + 8) + (R + 2 * D + Di)
    return {"append": B * append, "index_topk": B * topk, "sparse_decode": B * decode}


def _code_tokens(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed (the sources
    hold no string literal that contains a comment marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    """Digest of the code of the HIP sources (comments and layout excluded);
    traffic counters are reused only while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp4_compressed_sparse_csa2_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


# ------------------------------------------------------------------ GPU side
class Setup:
    def __init__(self, replicas: int, workload: str = WORKLOAD, keep_kv: bool = False):
        import torch

        import fp4_compressed_sparse_csa2_amd as csa2
        from harness import gen

        self.torch, self.csa2, self.gen = torch, csa2, gen
        dev = self.dev = torch.device("cuda:0")
        wl = self.wl = gen.WORKLOADS[workload]
        B, L, D, Di = wl.B, wl.L, wl.D, wl.Di
        self.lens = gen.ctx_lens(wl)
        pt, npages = gen.page_table(wl, self.lens)
        t0 = time.perf_counter()
        cache = csa2.Cache.allocate(B, pt.shape[1], npages, D, Di, torch.from_numpy(pt), dev)
        ring = np.zeros((B, gen.WINDOW, D), np.uint16)
        self.keys, self.tail, self.kv = [], [], []
        x_new = np.empty((B, D), np.uint16)
        k_new = np.empty((B, Di), np.int8)
        for b in range(B):
            Lb = int(self.lens[b])
            kv = gen.kv_bf16(wl, b, Lb)
            keys = gen.idx_keys(wl, b, Lb)
            csa2.quantize_append(cache, self.t(kv), torch.full((Lb,), b, dtype=torch.int32, device=dev),
                                 torch.arange(Lb, dtype=torch.int32, device=dev), keys=self.t(keys))
            ring[b] = gen.swa_ring(wl, kv, Lb)
            x_new[b], k_new[b] = kv[Lb - 1], keys[Lb - 1]
            self.keys.append(keys)
            if keep_kv:
                self.kv.append(kv)
            del kv
        torch.cuda.synchronize()
        log(f"cache built: {npages} pages of {cache.pages.shape[1]} B "
            f"({cache.pages.numel() / 2**20:.0f} MiB) in {time.perf_counter() - t0:.1f} s")
        self.ring_host = ring
        self.x_new, self.k_new = x_new, k_new
        ring_d = self.t(ring)
        self.caches = [cache] + [csa2.Cache(cache.pages.clone(), cache.page_table, D, Di)
                                 for _ in range(replicas - 1)]
        self.rings = [ring_d] + [ring_d.clone() for _ in range(replicas - 1)]
        self.ctx = self.t(self.lens.astype(np.int32))
        self.max_ctx = int(self.lens.max())
        self.q_idx_h, self.q_h = gen.idx_query(wl), gen.query(wl)
        self.q_idx, self.q = self.t(self.q_idx_h), self.t(self.q_h)
        self.sigma = float(gen.softmax_scale(wl))
        self.seq = torch.arange(B, dtype=torch.int32, device=dev)
        self.pos = self.t((self.lens - 1).astype(np.int32))
        self.xd, self.kd = self.t(x_new), self.t(k_new)
        self.idx = torch.empty((B, wl.K), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((B,), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, wl.H, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, wl.H), dtype=torch.float32, device=dev)
        self.ws_t, self.ws_d = csa2.Workspace(dev), csa2.Workspace(dev)
        torch.cuda.synchronize()

    def t(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)

    # the three library calls of one step, on replica r
    def append(self, r):
        self.csa2.quantize_append(self.caches[r], self.xd, self.seq, self.pos, keys=self.kd,
                                  swa=self.rings[r])

    def index_topk(self, r):
        self.csa2.index_topk(self.caches[r], self.ctx, self.max_ctx, self.q_idx, self.wl.K,
                             self.ws_t, out_idx=self.idx, out_count=self.cnt)

    def decode(self, r):
        self.csa2.sparse_decode(self.caches[r], self.ctx, self.q, self.sigma, self.idx, self.cnt,
                                self.rings[r], self.ws_d, out=self.out, lse=self.lse)

    def append_index_topk(self, r):
        self.csa2.append_index_topk(self.caches[r], self.xd, self.seq, self.pos, self.kd,
                                    self.rings[r], self.ctx, self.max_ctx, self.q_idx, self.wl.K,
                                    self.ws_t, out_idx=self.idx, out_count=self.cnt)

    def step(self, r):
        """One decode step: the append fused into the Full layer's selection, then attention."""
        self.append_index_topk(r)
        self.decode(r)

    def step_unfused(self, r):
        """The same step as three separate calls."""
        self.append(r)
        self.index_topk(r)
        self.decode(r)


def capture(S: Setup, fn, rs):
    """HIP graph of fn(r) for r in rs on a side stream (torch's capture stream)."""
    torch = S.torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in rs:
            fn(r)
    return g


def time_call(S: Setup, fn, R: int, reps: int = 20) -> float:
    """Microseconds per call of fn(r): a graph of 4 rounds over the R replicas,
    replayed reps times between HIP events on the stream it runs on."""
    torch = S.torch
    g = capture(S, fn, [r for _ in range(4) for r in range(R)])
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * 4 * R)


def copy_gbs(torch, nbytes: int = 1 << 30) -> float:
    """Device-to-device copy rate (read + write bytes per second) of a plain
    torch copy: the stream reference the roofline fraction can be read against."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / 5
    del a, b
    return 2 * nbytes / t / 1e9


def read_gbs(torch, csa2, nbytes: int = 2 << 30) -> float:
    """Rate of the library's read-only stream kernel (csa2_stream_read, 16-byte
    non-temporal loads) over a buffer far larger than the last-level cache:
    the in-run reference for a read-bound kernel on this HBM."""
    a = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    csa2.stream_read(a, sink)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        csa2.stream_read(a, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / 10
    del a
    return nbytes / t / 1e9


def chain_calls(S: Setup) -> dict:
    """The Reindex / Reuse rows timed on this cache, with the shapes of the
    three-layer chain workload: a Full Top-K pool of 8192, a Reindex layer
    refiltering it to 2048 with its own indexer query, and the decodes of the
    Reindex layer and of a Reuse layer (own queries, same indices)."""
    torch, csa2, gen = S.torch, S.csa2, S.gen
    wl, dev, R = S.wl, S.dev, len(S.caches)
    wlc = gen.WORKLOADS["chain_64k"]
    B, Kf, K2 = wl.B, wlc.K, wlc.K2
    pool = torch.empty((B, Kf), dtype=torch.int32, device=dev)
    pc = torch.empty((B,), dtype=torch.int32, device=dev)
    idx2 = torch.empty((B, K2), dtype=torch.int32, device=dev)
    c2 = torch.empty((B,), dtype=torch.int32, device=dev)
    q1 = S.t(gen.idx_query(wlc, 1))
    qa, qb = S.t(gen.query(wlc, 1)), S.t(gen.query(wlc, 2))
    outs = [torch.empty((B, wl.H, wl.D), dtype=torch.float32, device=dev) for _ in range(2)]
    lses = [torch.empty((B, wl.H), dtype=torch.float32, device=dev) for _ in range(2)]
    ws = [csa2.Workspace(dev) for _ in range(4)]
    sigma = float(gen.softmax_scale(wlc))

    q0 = S.t(gen.query(wlc, 0))
    out_f = torch.empty((B, wl.H, wl.D), dtype=torch.float32, device=dev)
    lse_f = torch.empty((B, wl.H), dtype=torch.float32, device=dev)
    ws_f = csa2.Workspace(dev)

    def full(r):
        csa2.index_topk(S.caches[r], S.ctx, S.max_ctx, S.q_idx, Kf, ws[0], out_idx=pool,
                        out_count=pc)

    def dec_full_layer(r):
        csa2.sparse_decode(S.caches[r], S.ctx, q0, sigma, pool, pc, S.rings[r], ws_f,
                           out=out_f, lse=lse_f)

    def reindex(r):
        csa2.reindex(S.caches[r], q1, pool, pc, K2, ws[1], out_idx=idx2, out_count=c2)

    def dec_reindex_layer(r):
        csa2.sparse_decode(S.caches[r], S.ctx, qa, sigma, idx2, c2, S.rings[r], ws[2],
                           out=outs[0], lse=lses[0])

    def dec_reuse_layer(r):
        csa2.sparse_decode(S.caches[r], S.ctx, qb, sigma, idx2, c2, S.rings[r], ws[3],
                           out=outs[1], lse=lses[1])

    def chain_step(r):
        """The three layers' hot path in order: Full selection and attention,
        Reindex refilter and attention, Reuse attention."""
        full(r)
        dec_full_layer(r)
        reindex(r)
        dec_reindex_layer(r)
        dec_reuse_layer(r)

    for r in range(R):                       # eager pass sizes the workspaces
        chain_step(r)
    torch.cuda.synchronize()
    t = {name: time_call(S, fn, R) for name, fn in (
        ("full_index_topk_8192", full), ("sparse_decode_full_layer_8192", dec_full_layer),
        ("reindex_8192_to_2048", reindex),
        ("sparse_decode_reindex_layer", dec_reindex_layer),
        ("sparse_decode_reuse_layer", dec_reuse_layer), ("chain_step", chain_step))}
    L = S.max_ctx
    rbytes = B * (Kf * (4 + wl.Di) + wl.Di + 4 * K2)
    full_b = algorithmic_bytes(B, L, wl.H, wl.D, wl.Di, Kf)
    dec2 = algorithmic_bytes(B, L, wl.H, wl.D, wl.Di, K2)["sparse_decode"]
    step_bytes = full_b["index_topk"] + full_b["sparse_decode"] + rbytes + 2 * dec2
    return {"workload": "chain_64k on the b8_64k cache: Full layer (Top-K 8192 and its "
                        "decode over the 8192) -> Reindex layer (Top-K 2048 of the pool and "
                        "its decode) -> Reuse layer (decode over the Reindex indices)",
            "calls_us": t,
            "step_us": t["chain_step"],
            "layer_queries_per_s": 3 * B / (t["chain_step"] * 1e-6),
            "step_bytes": step_bytes,
            "step_gbs": step_bytes / (t["chain_step"] * 1e-6) / 1e9,
            "full_decode_8192_gbs": full_b["sparse_decode"]
                                    / (t["sparse_decode_full_layer_8192"] * 1e-6) / 1e9,
            "reindex_layer_step_us": t["reindex_8192_to_2048"] + t["sparse_decode_reindex_layer"],
            "reuse_layer_step_us": t["sparse_decode_reuse_layer"],
            "reindex_algorithmic_bytes": rbytes,
            "reindex_gbs": rbytes / (t["reindex_8192_to_2048"] * 1e-6) / 1e9}


def ragged_calls(reps: int = 10) -> dict:
    """The 128-sequence ragged workload (contexts U{8192..131072}, 64-token
    pages through one global random permutation, every sequence appending one
    token per step): the step as the headline step runs it (the append fused
    into the indexer's scoring launch, then attention) and as its three
    separate calls, each call's time and rate.
    Its 3.5 GB cache is far larger than the 256 MB last-level cache, so one
    replica suffices.  The decode call moves 118 MB here, enough to price it
    against the HBM roofline on its own."""
    S = Setup(1, "b128_rag")
    torch, wl = S.torch, S.wl
    S.step_unfused(0)
    S.step(0)
    torch.cuda.synchronize()
    calls = {name: time_call(S, fn, 1, reps=reps) for name, fn in (
        ("append", S.append), ("index_topk", S.index_topk),
        ("append_index_topk", S.append_index_topk), ("sparse_decode", S.decode),
        ("step", S.step), ("step_unfused", S.step_unfused))}
    nb = {"append": 0, "index_topk": 0, "sparse_decode": 0}
    for L in S.lens:
        for k, v in algorithmic_bytes(1, int(L), wl.H, wl.D, wl.Di, wl.K).items():
            nb[k] += v
    step_bytes = sum(nb.values())
    dec_flops = 4 * wl.H * wl.D * (wl.K + 128) * wl.B
    gbs = {k: nb[k] / (calls[k] * 1e-6) / 1e9 for k in nb}
    res = {"workload": "b128_rag: batch 128, ctx U{8192..131072} (total "
                       f"{int(S.lens.sum())} tokens), 64-token pages in a permuted page table, "
                       "64 heads, latent 512 FP4, indexer dim 128, Top-K 2048, SWA 128; step = "
                       "append_index_topk (one token per sequence appended in the scoring "
                       "launch) + sparse_decode; step_unfused = quantize_append + index_topk "
                       "+ sparse_decode",
           "calls_us": calls,
           "queries_per_s": wl.B / (calls["step"] * 1e-6),
           "step_bytes": step_bytes,
           "step_gbs": step_bytes / (calls["step"] * 1e-6) / 1e9,
           "calls_bytes": nb,
           "calls_gbs": gbs,
           "sparse_decode_hbm_frac": gbs["sparse_decode"] / HBM_PEAK_GBS,
           "sparse_decode_mfma_frac": dec_flops / (calls["sparse_decode"] * 1e-6) / 1e12
                                      / MFMA_F16_PEAK_TFLOPS,
           "index_topk_hbm_frac": gbs["index_topk"] / HBM_PEAK_GBS}
    del S
    torch.cuda.empty_cache()
    return res


def long_context_calls(replicas: int = 3):
    """The one-sequence workload b1_1m (1,048,576 cached tokens, Top-K 2048,
    3-sigma boost of 1% of the keys) on one device: the step of the headline
    (append fused into the Full layer's selection, then attention) and its
    two calls, timed as graph replays over cold cache replicas (each about
    436 MB, together past the 256 MB last-level cache).  Returns the record
    and host copies of the eager step's results, which the CPU-oracle leg
    checks."""
    S = Setup(replicas, "b1_1m", keep_kv=True)
    torch, wl = S.torch, S.wl
    for r in range(replicas):
        S.step(r)
    torch.cuda.synchronize()
    eager = [t.cpu().numpy() for t in (S.idx, S.cnt, S.out, S.lse)]
    calls = {name: time_call(S, fn, replicas) for name, fn in (
        ("append_index_topk", S.append_index_topk), ("sparse_decode", S.decode),
        ("step", S.step))}
    L = int(S.lens.max())
    nb = algorithmic_bytes(1, L, wl.H, wl.D, wl.Di, wl.K)
    fused = nb["index_topk"] + nb["append"]
    step_bytes = sum(nb.values())
    fused_gbs = fused / (calls["append_index_topk"] * 1e-6) / 1e9
    res = {"workload": f"b1_1m: batch 1, ctx {L}, 64 heads, latent 512 FP4, indexer dim 128, "
                       "Top-K 2048, SWA 128, 3-sigma boost of 1% of the keys",
           "calls_us": calls,
           "queries_per_s": 1.0 / (calls["step"] * 1e-6),
           "step_bytes": step_bytes,
           "step_gbs": step_bytes / (calls["step"] * 1e-6) / 1e9,
           "step_hbm_frac": step_bytes / (calls["step"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
           "roofline": {"kernel": "csa2_append_index_topk", "bound": "hbm",
                        "achieved": fused_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": fused_gbs / HBM_PEAK_GBS, "bytes_per_launch": fused,
                        "launch_us": calls["append_index_topk"]},
           "sparse_decode_gbs": nb["sparse_decode"] / (calls["sparse_decode"] * 1e-6) / 1e9,
           "parity": "skipped (checked in the CPU-oracle leg)"}
    check = {"q_idx": S.q_idx_h[0], "keys": S.keys[0], "kv": S.kv[0], "q": S.q_h[0],
             "ring": S.ring_host[0], "sigma": S.sigma, "L": L, "K": wl.K, "gpu": eager}
    del S
    torch.cuda.empty_cache()
    return res, check


def scaled_calls(S: Setup) -> dict:
    """The scaled indexer (a fp32 key scale per token, ranked by
    fl32(s * score)) at the step's shape: the Full layer's Top-K 2048 and a
    Reindex 8192 -> 2048 over a scaled pool.  Returns the record and the
    Full layer's selection of sequence 0 with its key scales, which the
    CPU-oracle leg checks."""
    torch, csa2, gen = S.torch, S.csa2, S.gen
    wl, dev, R = S.wl, S.dev, len(S.caches)
    B, K, Kf = wl.B, wl.K, gen.WORKLOADS["chain_64k"].K
    host = [gen.key_scales(wl, b, int(S.lens[b])) for b in range(B)]
    ks = [csa2.key_scales_for(c) for c in S.caches]
    for b in range(B):
        Lb = int(S.lens[b])
        sb, pb = torch.full((Lb,), b, dtype=torch.int32, device=dev), \
            torch.arange(Lb, dtype=torch.int32, device=dev)
        for r in range(R):
            csa2.store_key_scales(S.caches[r], S.t(host[b]), sb, pb, ks[r])
    idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    cnt = torch.empty((B,), dtype=torch.int32, device=dev)
    pool = torch.empty((B, Kf), dtype=torch.int32, device=dev)
    pc = torch.empty((B,), dtype=torch.int32, device=dev)
    q1 = S.t(gen.idx_query(gen.WORKLOADS["chain_64k"], 1))
    ws = [csa2.Workspace(dev) for _ in range(3)]

    def topk(r):
        csa2.index_topk_scaled(S.caches[r], S.ctx, S.max_ctx, S.q_idx, ks[r], K, ws[0],
                               out_idx=idx, out_count=cnt)

    def full_pool(r):
        csa2.index_topk_scaled(S.caches[r], S.ctx, S.max_ctx, S.q_idx, ks[r], Kf, ws[1],
                               out_idx=pool, out_count=pc)

    def reindex(r):
        csa2.reindex_scaled(S.caches[r], q1, ks[r], pool, pc, K, ws[2], out_idx=idx,
                            out_count=cnt)

    topk(0)
    torch.cuda.synchronize()
    check = (idx[0].cpu().numpy(), int(cnt[0]), host[0])
    full_pool(0)
    reindex(0)
    torch.cuda.synchronize()
    t_topk = time_call(S, topk, R)
    t_full = time_call(S, full_pool, R)
    full_pool(0)
    torch.cuda.synchronize()
    t_re = time_call(S, reindex, R)
    L = int(S.lens.max())
    nbytes = algorithmic_bytes(B, L, wl.H, wl.D, wl.Di, K)["index_topk"] + B * 4 * (L - 128)
    return {"key_scales": "fp32 per token, exp(N(0,1))/128",
            "parity": "skipped (checked in the CPU-oracle leg)",
            "calls_us": {"index_topk_scaled_2048": t_topk, "index_topk_scaled_8192": t_full,
                         "reindex_scaled_8192_to_2048": t_re},
            "index_topk_scaled_bytes": nbytes,
            "index_topk_scaled_gbs": nbytes / (t_topk * 1e-6) / 1e9}, check


def gpu_bench(args, S: Setup):
    torch = S.torch
    R = args.replicas
    for r in range(R):                       # eager pass: sizes workspaces, checks results
        S.step(r)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (S.idx, S.cnt, S.out, S.lse)]

    per = max(1, 20 // R)                    # replicas x per steps in one graph
    big = capture(S, S.step, [r for _ in range(per) for r in range(R)])
    single = [capture(S, S.step, [r]) for r in range(R)]
    S_big = R * per

    def run_steps(k):
        for _ in range(k // S_big):
            big.replay()
        for j in range(k % S_big):
            single[j % R].replay()

    run_steps(args.warmup)
    torch.cuda.synchronize()
    for t, r in zip((S.idx, S.cnt, S.out, S.lse), ref):   # replays reproduce the eager result
        assert torch.equal(t, r), "graph replay differs from the eager step"

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    run_steps(args.steps)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1)

    # per-call durations: graphs of one call kind over the replicas
    calls = {name: time_call(S, fn, R) for name, fn in (
        ("append", S.append), ("index_topk", S.index_topk),
        ("append_index_topk", S.append_index_topk), ("sparse_decode", S.decode),
        ("step_unfused", S.step_unfused))}
    torch.cuda.synchronize()
    for t, r in zip((S.idx, S.cnt, S.out, S.lse), ref):
        assert torch.equal(t, r), "per-call replay differs from the eager step"

    # spread of the step time over replays of the big graph, and a warm step
    # (one replica, its keys resident in the last-level cache)
    per_step = []
    for _ in range(10):
        e0.record(stream)
        big.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per_step.append(e0.elapsed_time(e1) * 1e3 / S_big)
    warm_us = time_call(S, S.step, 1)
    # bounded replay: rebuild every window ring from the bf16 tokens of the
    # last 128 positions (csa2_quantize_append of B x 128 tokens, ring written)
    B, W = S.wl.B, 128
    seq = torch.arange(B, dtype=torch.int32, device=S.dev).repeat_interleave(W)
    pos = torch.cat([torch.arange(int(L) - W, int(L), dtype=torch.int32, device=S.dev)
                     for L in S.lens])
    tok = S.t(np.concatenate([S.ring_host[b][np.arange(int(L) - W, int(L)) % W]
                              for b, L in enumerate(S.lens)]))
    restore_us = time_call(S, lambda r: S.csa2.quantize_append(S.caches[r], tok, seq, pos,
                                                               swa=S.rings[r]), R)
    spread = {"p10": float(np.percentile(per_step, 10)), "p50": float(np.percentile(per_step, 50)),
              "p90": float(np.percentile(per_step, 90)), "warm_one_replica": warm_us,
              "replays": len(per_step), "steps_per_replay": S_big,
              "window_restore_us": restore_us}
    return wall, ev_ms, calls, spread, [t.cpu().numpy() for t in ref]


def schedule_calls(S: Setup, n_layers: int = 20) -> dict:
    """A decode step of an n-layer schedule on this cache: layer 0 Full with a
    pool of 8192, then per run of 4 layers one Reindex layer (Top-K' 2048 of
    the pool) and three Reuse layers of it; every layer with its own queries,
    the indexer layers with their own indexer queries.  Layers run in order
    (a layer's queries come from the previous layer's output)."""
    from fp4_compressed_sparse_csa2_amd.schedule import Runner, Schedule
    torch, gen = S.torch, S.gen
    wl, dev, R = S.wl, S.dev, len(S.caches)
    sched = Schedule.pattern(n_layers, 8192, 2048, period=4)
    runners = [Runner(sched, S.caches[r]) for r in range(R)]
    q_idx = {i: S.t(gen.idx_query(wl, i)) for i in sched.selecting_layers()}
    q = [S.t(gen.query(wl, i)) for i in range(n_layers)]
    outs = [torch.empty((wl.B, wl.H, wl.D), dtype=torch.float32, device=dev) for _ in range(n_layers)]
    lses = [torch.empty((wl.B, wl.H), dtype=torch.float32, device=dev) for _ in range(n_layers)]

    def step(r):
        runners[r].step(S.ctx, S.max_ctx, q_idx, q, [S.rings[r]] * n_layers, S.sigma, outs, lses)

    for r in range(R):
        step(r)
    torch.cuda.synchronize()
    t = time_call(S, step, R, reps=5)
    modes = [l.mode for l in sched.layers]
    return {"schedule": f"{n_layers} layers: " + ", ".join(f"{modes.count(m)} {m}" for m in
                                                             ("full", "reindex", "reuse")),
            "step_us": t, "us_per_layer": t / n_layers,
            "layer_queries_per_s": wl.B * n_layers / (t * 1e-6)}


# ------------------------------------------------------------------ sharded context
def shard_bounds(L: int, n: int) -> list:
    """n page-aligned ascending position ranges covering [0, L); the last is open."""
    pages = -(-L // 64)
    cuts = [int(round(pages * i / n)) * 64 for i in range(n)]
    return [(cuts[i], cuts[i + 1] if i + 1 < n else 1 << 24) for i in range(n)]


def dcp_bench(args) -> dict:
    """The 1M-token sequence cut into N page-aligned shards, one per emulated
    device: each shard's range Top-K (with scores), the merge of the shard
    lists, each shard's attention over the merged selection through a page
    table that holds only its pages (the window on the tail shard), and the
    LSE merge; against the one-device index_topk + sparse_decode on the same
    cache.  Calls are timed as graph replays over two cold cache replicas.
    The emulated step adds the slowest shard's selection, the merge, the
    slowest shard's decode and the LSE merge; the exchanges between devices
    (an all-gather of N*K (score, position) pairs and a reduction of the
    partial outputs) are not part of it."""
    import torch
    S = Setup(2, "b1_1m")
    csa2, wl, dev = S.csa2, S.wl, S.dev
    n, B, K, H, D = args.dcp, wl.B, wl.K, wl.H, wl.D
    L = int(S.lens.max())
    bounds = shard_bounds(L, n)
    R = len(S.caches)
    pidx = torch.empty((n, B, K), dtype=torch.int32, device=dev)
    psc = torch.empty((n, B, K), dtype=torch.int32, device=dev)
    pcnt = torch.empty((n, B), dtype=torch.int32, device=dev)
    midx = torch.empty((B, K), dtype=torch.int32, device=dev)
    mcnt = torch.empty((B,), dtype=torch.int32, device=dev)
    msc = torch.empty((B, K), dtype=torch.int32, device=dev)
    outs = torch.empty((n, B, H, D), dtype=torch.float32, device=dev)
    lses = torch.empty((n, B, H), dtype=torch.float32, device=dev)
    out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws_t = [csa2.Workspace(dev) for _ in range(n)]
    ws_d = [csa2.Workspace(dev) for _ in range(n)]
    ws_m = csa2.Workspace(dev)
    views = []
    for r in range(R):
        vs = []
        for s, (a, e) in enumerate(bounds):
            pt = S.caches[r].page_table.clone()
            own = torch.zeros(pt.shape[1], dtype=torch.bool, device=dev)
            own[a // 64: min(pt.shape[1], -(-e // 64))] = True
            pt[:, ~own] = -1
            vs.append(csa2.Cache(S.caches[r].pages, pt.contiguous(), D, wl.Di))
        views.append(vs)

    def topk_fn(s):
        a, e = bounds[s]
        return lambda r: csa2.index_topk_range(S.caches[r], S.ctx, S.max_ctx, S.q_idx, K, a, e,
                                               ws_t[s], out_idx=pidx[s], out_count=pcnt[s],
                                               out_sel_scores=psc[s])

    def merge(r):
        csa2.topk_merge(pidx, psc, pcnt, K, ws_m, out_idx=midx, out_count=mcnt, out_sel_scores=msc)

    def dec_fn(s):
        return lambda r: csa2.sparse_decode(views[r][s], S.ctx, S.q, S.sigma, midx, mcnt,
                                            S.rings[r] if s == n - 1 else None, ws_d[s],
                                            out=outs[s], lse=lses[s])

    def lsem(r):
        csa2.lse_merge(outs, lses, out=out, lse=lse)

    for r in range(R):                        # eager pass: workspaces, results
        for s in range(n):
            topk_fn(s)(r)
        merge(r)
        for s in range(n):
            dec_fn(s)(r)
        lsem(r)
        S.index_topk(r)
        S.decode(r)
    torch.cuda.synchronize()
    same_idx = bool(torch.equal(midx, S.idx) and torch.equal(mcnt, S.cnt))
    out_err = float((out - S.out).abs().max())
    t_topk = [time_call(S, topk_fn(s), R) for s in range(n)]
    t_merge = time_call(S, merge, R)
    t_dec = [time_call(S, dec_fn(s), R) for s in range(n)]
    t_lse = time_call(S, lsem, R)
    t_one_topk = time_call(S, S.index_topk, R)
    t_one_dec = time_call(S, S.decode, R)
    emulated = max(t_topk) + t_merge + max(t_dec) + t_lse
    one = t_one_topk + t_one_dec
    return {"metric": "context-sharded decode step, emulated on one GPU",
            "workload": f"b1_1m: batch 1, ctx {L}, 64 heads, latent 512 FP4, indexer dim 128, "
                        f"Top-K {K}, SWA 128; {n} page-aligned shards",
            "shards": [list(b) for b in bounds],
            "range_topk_us": t_topk, "merge_us": t_merge, "shard_decode_us": t_dec,
            "lse_merge_us": t_lse, "emulated_step_us": emulated,
            "one_device": {"index_topk_us": t_one_topk, "sparse_decode_us": t_one_dec,
                           "step_us": one},
            "speedup_vs_one_device": one / emulated,
            "merged_indices_equal_one_device": same_idx,
            "merged_out_max_abs_diff_vs_one_device": out_err,
            "excluded": "device-to-device exchanges (all-gather of N*K pairs, reduction of "
                        "the partial outputs)"}


# ------------------------------------------------------------------ CPU oracle
def scaled_parity(S: Setup, check) -> str:
    """The scaled indexer's Top-K of sequence 0 (from scaled_calls) against
    the oracle's ranking of fl32(s * score)."""
    from oracle import select as OS

    got, got_cnt, scales = check
    L0 = int(S.lens[0])
    v = OS.scaled_values(OS.indexer_scores(S.q_idx_h[0], S.keys[0][:L0 - 128]), scales[:L0 - 128])
    want, wc, _ = OS.topk_values(v, L0, S.wl.K)
    assert got_cnt == wc and np.array_equal(got, want), "scaled Top-K differs from the oracle, b=0"
    return "ok (sequence 0 against the oracle: Top-K bit-exact)"


def long_context_parity(check) -> str:
    """The b1_1m eager step against the oracle: Top-K bit-exact, outputs and
    LSE within 2e-3."""
    from oracle import attention as OA
    from oracle import formats as OF
    from oracle import select as OS

    L, K = check["L"], check["K"]
    g_idx, g_cnt, g_out, g_lse = (t[0] for t in check["gpu"])
    idx, c = OS.topk(OS.indexer_scores(check["q_idx"], check["keys"][:L - 128]), L, K)
    assert int(g_cnt) == c and np.array_equal(g_idx, idx), "b1_1m Top-K differs from the oracle"
    sel = idx[:c]
    o, lse = OA.sparse_decode(check["q"], check["sigma"], *OF.quantize_rows(check["kv"][sel]),
                              check["ring"], sel, L)
    err = max(float(np.max(np.abs(g_out - o))), float(np.max(np.abs(g_lse - lse))))
    assert err <= 2e-3, f"b1_1m attention error {err:.3e}"
    return f"ok (the sequence against the oracle: Top-K bit-exact, max-abs error {err:.1e})"


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(S: Setup, seconds: float, gpu=None):
    """The oracle's decode step (append of the new token, indexer scores,
    Top-K, dequantisation of the selected rows, merged attention) on the same
    seeded sequences, repeated until ``seconds`` of timed work.  Every
    sequence runs at least once; with ``gpu`` (host copies of the GPU step's
    idx, count, out, lse) the first run of each sequence is also compared
    with it, outside the timed parts: indices bit-exact, outputs and LSE
    within 2e-3.  Returns (baseline record, parity string)."""
    import threadpoolctl

    from oracle import attention as OA
    from oracle import formats as OF
    from oracle import select as OS

    wl = S.wl
    K = wl.K
    stored = {}                       # the oracle cache's rows at each sequence's selection
    worst, checked = 0.0, set()
    done, timed = 0, 0.0
    b = 0
    while timed < seconds or done < wl.B:
        L = int(S.lens[b])
        t0 = time.perf_counter()
        OF.quantize_rows(S.x_new[b:b + 1])                      # append of the new token
        sc = OS.indexer_scores(S.q_idx_h[b], S.keys[b][:L - 128])
        idx, c = OS.topk(sc, L, K)
        t1 = time.perf_counter()
        sel = idx[:c]
        if b not in stored:           # cache content (written at prefill), not part of the step
            stored[b] = OF.quantize_rows(S.gen.kv_bf16(wl, b, L)[sel])
        t2 = time.perf_counter()
        o, lse = OA.sparse_decode(S.q_h[b], S.sigma, *stored[b], S.ring_host[b], sel, L)
        t3 = time.perf_counter()
        timed += (t1 - t0) + (t3 - t2)
        if gpu is not None and b not in checked:
            g_idx, g_cnt, g_out, g_lse = (t[b] for t in gpu)
            assert int(g_cnt) == c and np.array_equal(g_idx, idx), f"Top-K differs, b={b}"
            err = max(float(np.max(np.abs(g_out - o))), float(np.max(np.abs(g_lse - lse))))
            assert err <= 2e-3, f"attention error {err:.3e}, b={b}"
            worst = max(worst, err)
            checked.add(b)
        done += 1
        b = (b + 1) % wl.B
    info = threadpoolctl.threadpool_info()
    threads = max([1] + [int(i.get("num_threads", 1)) for i in info])
    L = int(S.lens.max())
    per_query = sum(algorithmic_bytes(1, L, wl.H, wl.D, wl.Di, K).values())
    parity = ("skipped" if gpu is None else
              f"ok (all {wl.B} sequences against the oracle: Top-K bit-exact, "
              f"max-abs error {worst:.1e})")
    return {"value": done / timed, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "gbs": done / timed * per_query / 1e9,
            "sample": f"{done} whole decode steps (sequences of {WORKLOAD} in turn), "
                      f"{timed:.1f} s of timed oracle work; numpy float64, BLAS threads {threads}",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}, parity


# ------------------------------------------------------------------ counters
CALIB_BYTES = 1 << 30
STEP_KERNELS = {"append_index_topk": ("append_score_kernel", "select_single_kernel",
                                      "select_filter_kernel", "select_final_kernel"),
                "sparse_decode": ("sparse_decode_kernel", "sparse_combine_kernel")}


def counter_run(args) -> int:
    """Device copies of a known size, then eager steps, for the counter passes
    (the b8_64k step, or with --ragged-only the b128_rag step as its three
    calls)."""
    import torch
    a = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda:0")
    bb = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        bb.copy_(a)
    torch.cuda.synchronize()
    del a, bb
    if args.ragged_only:
        S = Setup(1, "b128_rag")
        for i in range(args.warmup + args.steps):
            S.step_unfused(0)
    else:
        S = Setup(args.replicas)
        for i in range(args.warmup + args.steps):
            S.step(i % args.replicas)
    torch.cuda.synchronize()
    print(json.dumps({"counter_run": True, "steps": args.steps, "calib_bytes": CALIB_BYTES,
                      "calib_copies": 3}), flush=True)
    return 0


def _read_counters(d: str, counter: str):
    """{dispatch id: (kernel name, value)} for one counter from a rocprofv3 --pmc output dir."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    out = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (fn, int(row["Dispatch_Id"]))
                name, val = out.get(key, (row["Kernel_Name"], 0.0))
                out[key] = (name, val + float(row["Counter_Value"]))
    return out


def traffic_from(fetch_dir: str, write_dir: str, steps: int) -> dict:
    """Bytes per launch of each library call from the FETCH_SIZE / WRITE_SIZE
    passes, each scaled by what the counter reads for a 1 GiB device copy."""
    res = {"source_digest": source_digest(), "kernels": {}, "calibration": {}}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        recs = _read_counters(d, counter)
        ordered = [recs[k] for k in sorted(recs, key=lambda k: k[1])]
        # the calibration copies are the only copy dispatches of this size class
        # (FETCH_SIZE reads a 1 GiB copy as about half of it on gfx950)
        big = [v for n, v in ordered if "copy" in n.lower() and v * 1024 > 0.25 * CALIB_BYTES]
        if not big:
            raise SystemExit(f"{counter}: no calibration copy found")
        calib_kib = float(np.median(big))
        factor = CALIB_BYTES / (calib_kib * 1024.0)
        res["calibration"][counter] = {"copy_bytes": CALIB_BYTES, "reads_kib": calib_kib,
                                       "factor": factor}
        for call, kernels in STEP_KERNELS.items():
            tot = 0.0
            for kname in kernels:
                vals = [v for n, v in ordered if kname in n][-steps:]
                if vals:
                    tot += float(np.mean(vals)) * 1024.0 * factor
                    per.setdefault(kname, {})[counter] = float(np.mean(vals)) * 1024.0 * factor
            per.setdefault(call, {})[counter] = tot
    for name, v in per.items():
        v["bytes_per_launch"] = v.get("FETCH_SIZE", 0.0) + v.get("WRITE_SIZE", 0.0)
        res["kernels"][name] = v
    return res


# Kernel sequences of one step per workload in a trace of the default run:
# (title, kernel-name patterns in launch order, grid rows of the first kernel).
TRACE_STEPS = [
    ("b8_64k step: csa2_append_index_topk + csa2_sparse_decode",
     [r"append_score_kernel<512, 128, \d+>", r"select_filter_kernel<IntKeys>",
      r"select_final_kernel<\d+, IntKeys, false>", r"sparse_decode_kernel<512, 16, true>",
      r"sparse_combine_kernel<512, 16, \d+>"], 9),
    ("b1_1m step: csa2_append_index_topk + csa2_sparse_decode",
     [r"append_score_kernel<512, 128, \d+>", r"select_filter_kernel<IntKeys>",
      r"select_final_kernel<\d+, IntKeys, false>", r"sparse_decode\w*_kernel<512[^>]*>",
      r"sparse_combine_kernel<512, \d+, \d+>"], 2),
    ("b128_rag csa2_index_topk",
     [r"index_score_kernel<128, false, \d+>", r"select_filter_kernel<IntKeys>",
      r"select_final_kernel<\d+, IntKeys, false>"], 128),
    ("b128_rag csa2_sparse_decode",
     [r"sparse_decode64_kernel<512>", r"sparse_combine_kernel<512, 64, \d+>"], None),
    ("b8_64k csa2_reindex 8192 -> 2048",
     [r"reindex_score_kernel<128, false>", r"select_single_kernel<IntKeys, true>"], None),
]


def trace_summary(path: str) -> str:
    """Markdown tables of TRACE_STEPS from a rocprofv3 kernel-trace CSV:
    every run of the kernel sequence, per kernel the median duration and the
    median gap after the previous kernel, and the median whole run."""
    import csv
    import statistics
    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    names = [r["Kernel_Name"].split("(")[0].replace("void ", "").replace("csa2::", "")
             for r in rows]
    out = []
    for title, seq, grid_y in TRACE_STEPS:
        dur = [[] for _ in seq]
        gap = [[] for _ in seq]
        whole = []
        i = 0
        while i + len(seq) <= len(rows):
            if (all(re.fullmatch(seq[k], names[i + k]) for k in range(len(seq))) and
                    (grid_y is None or int(rows[i]["Grid_Size_Y"]) == grid_y)):
                g = rows[i:i + len(seq)]
                for k in range(len(seq)):
                    dur[k].append(int(g[k]["End_Timestamp"]) - int(g[k]["Start_Timestamp"]))
                    if k:
                        gap[k].append(int(g[k]["Start_Timestamp"]) - int(g[k - 1]["End_Timestamp"]))
                whole.append(int(g[-1]["End_Timestamp"]) - int(g[0]["Start_Timestamp"]))
                i += len(seq)
            else:
                i += 1
        out.append(f"{title}: {len(whole)} runs\n\n| kernel | median µs | median gap before µs |\n"
                   "|---|---|---|")
        for k in range(len(seq)):
            if dur[k]:
                g = f"{statistics.median(gap[k]) / 1e3:.2f}" if gap[k] else "-"
                out.append(f"| `{names_of(seq[k])}` | {statistics.median(dur[k]) / 1e3:.2f} | {g} |")
        if whole:
            out.append(f"| whole run | {statistics.median(whole) / 1e3:.2f} | |")
        out.append("")
    return "\n".join(out)


def names_of(pattern: str) -> str:
    return pattern.replace("\\d+", "N").replace("\\w*", "").replace("[^>]*", "...")


# ------------------------------------------------------------------ main
def main() -> int:
    args = parse()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return 0
    if args.traffic_from:
        rec = traffic_from(*args.traffic_from, args.steps)
        rec["command"] = ("rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv "
                          f"-- python3 bench.py --counter-run --steps {args.steps} "
                          f"--warmup {args.warmup}")
        path = os.path.join(ROOT, "profiles", "traffic.json")
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode step shards by sequence with no communication, so N GPUs "
              "would each run this same per-GPU workload).", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        return 2
    if args.counter_run:
        return counter_run(args)
    if args.ragged_only:
        print(json.dumps(ragged_calls()), flush=True)
        return 0
    if args.dcp:
        print(json.dumps(dcp_bench(args)), flush=True)
        return 0
    S = Setup(args.replicas)
    wl = S.wl
    wall, ev_ms, calls, spread, eager = gpu_bench(args, S)
    chain = scaled = ragged = scaled_check = long_ctx = long_check = None
    if not args.no_extras:
        chain = chain_calls(S)
        chain["schedule"] = schedule_calls(S)
        scaled, scaled_check = scaled_calls(S)
        log("b128_rag: building the ragged paged cache")
        ragged = ragged_calls()
        log("b1_1m: building the 1M-token cache")
        long_ctx, long_check = long_context_calls()
    copy_rate = copy_gbs(torch)
    read_rate = read_gbs(torch, S.csa2)
    B, L, H, D, Di, K = wl.B, int(S.lens.max()), wl.H, wl.D, wl.Di, wl.K
    nbytes = algorithmic_bytes(B, L, H, D, Di, K)
    step_bytes = sum(nbytes.values())
    step_s = ev_ms * 1e-3 / args.steps
    gbs = step_bytes / step_s / 1e9
    topk_gbs = nbytes["index_topk"] / (calls["index_topk"] * 1e-6) / 1e9
    fused_bytes = nbytes["index_topk"] + nbytes["append"]
    fused_gbs = fused_bytes / (calls["append_index_topk"] * 1e-6) / 1e9
    dec_gbs = nbytes["sparse_decode"] / (calls["sparse_decode"] * 1e-6) / 1e9
    dec_flops = 4 * H * D * (K + 128) * B                 # QK^T and PV over selected + window
    dec_tflops = dec_flops / (calls["sparse_decode"] * 1e-6) / 1e12
    traffic = measured_traffic("append_index_topk")
    res = {
        "metric": "decode attention queries/sec and achieved HBM GB/s (% of peak) at 64K ctx",
        "value": B / step_s,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8xi8->i32 indexer; fp4/bf16->f16 MFMA, f32 accumulate",
        "data": "synthetic (seeded bf16 N(0,1) latent rows, int8 uniform keys)",
        "config": {"workload": "b8_64k: batch 8, ctx 65536, 64 query heads over one latent-512 "
                               "FP4 E2M1/E4M3-per-16 KV (288 B/token), int8 indexer dim 128, "
                               "Top-K 2048 outside the last 128, bf16 SWA 128",
                   "batch": B, "ctx": L, "heads": H, "head_dim": D, "idx_dim": Di, "top_k": K,
                   "window": 128,
                   "step": "append_index_topk (the 1-token/seq quantize_append fused into the Full "
                           "layer's scoring launch, then the Top-K) + sparse_decode",
                   "replicas": args.replicas,
                   "timing": "HIP graph replays between HIP events on the kernels' stream"},
        "hbm_gbs": gbs,
        "hbm_frac_of_peak": gbs / HBM_PEAK_GBS,
        "step_bytes": step_bytes,
        "step_us_events": step_s * 1e6,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "sparse_decode_hbm_frac": dec_gbs / HBM_PEAK_GBS,
        "calls_us": calls,
        "calls_gbs": {"index_topk": topk_gbs, "append_index_topk": fused_gbs,
                      "sparse_decode": dec_gbs},
        "step_us_spread": spread,
        "sparse_decode_mfma": {"flops_per_call": dec_flops, "tflops": dec_tflops,
                               "peak_tflops": MFMA_F16_PEAK_TFLOPS,
                               "frac": dec_tflops / MFMA_F16_PEAK_TFLOPS},
        "copy_reference_gbs": copy_rate,
        "read_reference_gbs": read_rate,
        "chain": chain,
        "scaled_indexer": scaled,
        "ragged_b128": ragged,
        "long_b1_1m": long_ctx,
        "roofline": {"kernel": "csa2_append_index_topk ("
                               + ", ".join(STEP_KERNELS["append_index_topk"]) + ")",
                     "bound": "hbm", "achieved": fused_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": fused_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "frac_of_copy_reference": fused_gbs / copy_rate,
                     "frac_of_read_reference": fused_gbs / read_rate,
                     "launch_us": calls["append_index_topk"], "bytes_per_launch": fused_bytes},
        "parity": "skipped (checked in the CPU-oracle leg)",
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (and checking the GPU step against it)")
        res["cpu_baseline"], res["parity"] = cpu_baseline(
            S, args.cpu_seconds, None if args.no_parity else eager)
        log(f"parity: {res['parity']}")
        if scaled is not None and not args.no_parity:
            scaled["parity"] = scaled_parity(S, scaled_check)
        if long_ctx is not None and not args.no_parity:
            log("checking the b1_1m step against the oracle")
            long_ctx["parity"] = long_context_parity(long_check)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
