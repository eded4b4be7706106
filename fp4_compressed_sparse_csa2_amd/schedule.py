"""Static per-layer mode schedule and the owner/consumer cache graph.

Every attention layer is statically Full, Reindex or Reuse; the layers share
one main KV cache and one set of indexer keys, and Top-K addressing indices
are reused across layers (neodrop.ai V4.1-Flash report, 架构拆解 item 2).  A
Full layer builds the indexer state and selects; a Reindex layer keeps the KV
and recomputes the index over a pool; a Reuse layer consumes an earlier
layer's indices as they are (zulogic "DeepSeek V4 1-Flash 架构拆解",
section 3 mode table and owner/consumer diagram).  Readings where the pages
are silent: a Reindex layer refilters the pool of the nearest Full layer
before it (or the one it names), and a Reuse layer reuses the indices of the
nearest Full or Reindex layer before it (or the one it names).

A decode step runs the layers in order, because a layer's queries come from
the previous layer's output; what the schedule fixes is which index set each
layer attends over and which calls produce them.  The cache and the index
tensors are aliased, never copied: every layer passes the same Cache, and a
Reuse layer passes its source's (idx, count) tensors.
"""
from __future__ import annotations

import dataclasses
from typing import Sequence

import torch

from . import _lib

FULL, REINDEX, REUSE = "full", "reindex", "reuse"


@dataclasses.dataclass(frozen=True)
class Layer:
    mode: str                 # FULL, REINDEX or REUSE
    k: int = 0                # Top-K of a Full layer (its pool size) or Top-K' of a Reindex layer
    source: int | None = None  # the layer whose pool (Reindex) or indices (Reuse) this one uses


class Schedule:
    """A validated static schedule: for every layer, the layer whose indices
    it attends over (``index_owner``) and, for a Reindex layer, the Full layer
    whose pool it refilters (``pool_owner``)."""

    def __init__(self, layers: Sequence[Layer]):
        self.layers = list(layers)
        if not self.layers or self.layers[0].mode != FULL:
            raise ValueError("the first layer must be Full (it owns the indexer state)")
        self.index_owner: list[int] = []
        self.pool_owner: list[int | None] = []
        last_full = last_sel = None
        for i, l in enumerate(self.layers):
            if l.mode == FULL:
                if l.k < 1:
                    raise ValueError(f"layer {i}: a Full layer needs k >= 1")
                self.index_owner.append(i)
                self.pool_owner.append(None)
                last_full = last_sel = i
            elif l.mode == REINDEX:
                src = last_full if l.source is None else l.source
                if src is None or not (0 <= src < i) or self.layers[src].mode != FULL:
                    raise ValueError(f"layer {i}: a Reindex layer refilters an earlier Full layer's pool")
                if not (1 <= l.k <= self.layers[src].k):
                    raise ValueError(f"layer {i}: Top-K' must lie in [1, pool size {self.layers[src].k}]")
                self.index_owner.append(i)
                self.pool_owner.append(src)
                last_sel = i
            elif l.mode == REUSE:
                src = last_sel if l.source is None else l.source
                if src is None or not (0 <= src < i) or self.layers[src].mode == REUSE:
                    raise ValueError(f"layer {i}: a Reuse layer reuses an earlier Full or Reindex layer")
                self.index_owner.append(src)
                self.pool_owner.append(None)
            else:
                raise ValueError(f"layer {i}: unknown mode {l.mode!r}")

    @staticmethod
    def pattern(n_layers: int, k_full: int, k_reindex: int, period: int = 4) -> "Schedule":
        """Layer 0 Full; then, in every run of ``period`` layers, one Reindex
        layer of the Full layer's pool followed by Reuse layers of it."""
        layers = [Layer(FULL, k_full)]
        for i in range(1, n_layers):
            layers.append(Layer(REINDEX, k_reindex) if (i - 1) % period == 0 else Layer(REUSE))
        return Schedule(layers)

    def selecting_layers(self) -> list[int]:
        return [i for i, l in enumerate(self.layers) if l.mode != REUSE]


class Runner:
    """Runs one decode step of a schedule over one owner cache.  Holds the
    per-layer index tensors and workspaces (allocated on first use); the
    calls of a step go to torch's current stream in layer order."""

    def __init__(self, schedule: Schedule, cache: _lib.Cache):
        self.s, self.cache = schedule, cache
        dev, B = cache.device, cache.batch
        self.idx, self.cnt, self.ws = {}, {}, {}
        for i in schedule.selecting_layers():
            k = schedule.layers[i].k
            self.idx[i] = torch.empty((B, k), dtype=torch.int32, device=dev)
            self.cnt[i] = torch.empty((B,), dtype=torch.int32, device=dev)
            self.ws[i] = _lib.Workspace(dev)
        self.ws_dec = [_lib.Workspace(dev) for _ in schedule.layers]

    def indices(self, layer: int):
        """The (idx, count) tensors layer ``layer`` attends over (aliases for Reuse)."""
        o = self.s.index_owner[layer]
        return self.idx[o], self.cnt[o]

    def step(self, ctx_len: torch.Tensor, max_ctx: int, q_idx: dict, q: Sequence[torch.Tensor],
             swa: Sequence[torch.Tensor], softmax_scale: float, out: Sequence[torch.Tensor],
             lse: Sequence[torch.Tensor] | None = None) -> None:
        """q_idx[i]: the int8 indexer query of every Full / Reindex layer i;
        q[i], swa[i], out[i] (and lse[i]): every layer's queries, window ring
        and outputs."""
        for i, l in enumerate(self.s.layers):
            if l.mode == FULL:
                _lib.index_topk(self.cache, ctx_len, max_ctx, q_idx[i], l.k, self.ws[i],
                                out_idx=self.idx[i], out_count=self.cnt[i])
            elif l.mode == REINDEX:
                src = self.s.pool_owner[i]
                _lib.reindex(self.cache, q_idx[i], self.idx[src], self.cnt[src], l.k, self.ws[i],
                             out_idx=self.idx[i], out_count=self.cnt[i])
            idx, cnt = self.indices(i)
            _lib.sparse_decode(self.cache, ctx_len, q[i], softmax_scale, idx, cnt, swa[i],
                               self.ws_dec[i], out=out[i], lse=None if lse is None else lse[i])
