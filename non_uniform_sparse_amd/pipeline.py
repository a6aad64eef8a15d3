"""One decode step over every layer of a workload, on one GPU.

Set-up (once): cluster heads by budget, build the ragged caches and their
min-max metadata, plan the static split map, allocate the step's buffers.
Step: for each layer, [score pages -> top-K pages ->] split-K decode +
combine, all launched with no host synchronisation; the grid of every
launch comes from the static split map, never from the data.

Micro-batches.  Requests are independent, so the batch can be cut into
parts whose layer chains run on streams of their own, captured as one
graph (fork, one chain per stream, join).  One part's latency-bound phases
(top-K, kernel boundaries, the ramp and tail of each kernel) then overlap
another part's HBM-bound ones.  Every request gets the same split row S[l]
either way, so its result is the same bit for bit.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import kvs
from .layout import RaggedLayout, build_caches
from .workloads import Workload, torch_dtype

__all__ = ["DecodeStep", "splits_per_request", "topk_cap", "default_microbatches"]


def splits_per_request(W: int, b: int, G: int, mean_units: float, min_units: int = 4) -> int:
    """Splits T of one request's layer: enough workgroups to fill the chip
    (W concurrent, shared by b requests), but no split smaller than about
    ``min_units`` pages and never fewer than one split per group.  The floor
    only binds for small batches of short requests (measured on a one-request
    step: 4 pages per split 12% faster than 8; 2 no faster than 4)."""
    t = W // max(1, b)
    t = min(t, max(1, math.ceil(mean_units / min_units)))
    return max(G, t)


def default_microbatches(wl: Workload) -> int:
    """Request micro-batches for the step graph.  Parts only overlap once
    their layer chains drift apart; with a single layer (or a few) every part
    runs the same phase at the same time and the split only adds launches
    (measured: one-layer steps are fastest unsplit; the 32- and 48-layer
    steps fastest with 2 parts, 1-2% ahead of 3 and further ahead of 4)."""
    c = wl.cfg
    return 1 if c.L < 4 else min(2, c.b)


def topk_cap(wl: Workload) -> float:
    """Budget cap for the split weights when a top-K also bounds the work:
    a head never attends more than K*P tokens, i.e. a budget of K*P / N.
    The map has no request axis, and the longest request of the batch sets
    the launch's duration, so N is the longest context: the cap is the
    budget at which a head of that request attends all of its K pages."""
    c = wl.cfg
    if not c.topk:
        return 0.0
    return min(1.0, c.topk * c.P / float(wl.contexts.max()))


def fused_selection(wl: Workload, spread: float = 1.25) -> List[bool]:
    """Per layer: score and select in one launch (one workgroup per head,
    kvs_select_pages) when every head of the layer holds pages and the
    longest holds at most ``spread`` times the mean; otherwise the
    resident-grid scoring kernel balances the ragged heads and the top-K
    runs as a launch of its own."""
    c = wl.cfg
    if not c.topk:
        return [False] * c.L
    npg = -(-wl.n // c.P)
    return [bool(npg[:, l].min() > 0 and npg[:, l].max() <= spread * npg[:, l].mean())
            for l in range(c.L)]


@dataclass
class LayerBuffers:
    scores: Optional[torch.Tensor]
    sel: Optional[torch.Tensor]
    sel_count: Optional[torch.Tensor]
    out: torch.Tensor


class DecodeStep:
    def __init__(self, wl: Workload, device="cuda", T: Optional[int] = None,
                 head_slot: Optional[np.ndarray] = None, S: Optional[np.ndarray] = None,
                 poison: bool = True, microbatches: int = 1, growth: int = 0,
                 fused: Optional[bool] = None):
        c = wl.cfg
        self.wl, self.cfg, self.device = wl, c, device
        if head_slot is None:
            head_slot = (kvs.kvs_cluster_heads(wl.budgets, c.Hp) if c.clustered else
                         np.tile(np.arange(c.Hkv, dtype=np.int32), (c.L, 1)))
        self.head_slot = np.asarray(head_slot, dtype=np.int32)
        self.caches, self.layouts = build_caches(wl, self.head_slot, device=device, poison=poison,
                                                 growth=growth)
        for cache in self.caches:
            kvs.kvs_build_minmax(cache)
        dt = torch_dtype(c.dtype)
        self.W = kvs.kvs_decode_concurrency(torch.device(device).index or 0, c.d, c.Gq, dt)
        if S is None:
            if T is None:
                if c.topk:
                    units = float(np.minimum(c.topk, -(-wl.n // c.P)).sum(axis=2).mean())
                else:
                    units = float((-(-wl.n // c.P)).sum(axis=2).mean())
                T = splits_per_request(self.W, c.b, c.G, units)
            S = kvs.kvs_plan_split(wl.budgets, self.head_slot, c.Hp, topk_cap(wl), T)
        self.scale = 1.0 / math.sqrt(c.d)
        self.fused = fused_selection(wl) if fused is None else [bool(fused and c.topk)] * c.L
        self.set_splits(S, microbatches)
        self.bufs: List[LayerBuffers] = []
        for l in range(c.L):
            maxpg = self.layouts[l].page_table.shape[2]
            if c.topk:
                scores = torch.empty((c.b, c.Hkv, maxpg), dtype=torch.float32, device=device)
                sel = torch.empty((c.b, c.Hkv, c.topk), dtype=torch.int32, device=device)
                cnt = torch.empty((c.b, c.Hkv), dtype=torch.int32, device=device)
            else:
                scores = sel = cnt = None
            out = torch.empty((c.b, c.Hq, c.d), dtype=torch.float32, device=device)
            self.bufs.append(LayerBuffers(scores, sel, cnt, out))

    def set_splits(self, S, microbatches: Optional[int] = None) -> None:
        """Use the split map S [L][G] (T = its row sum per request) and size
        the decode workspaces for it, whole-batch and per micro-batch."""
        c, device = self.cfg, self.device
        self.S = np.asarray(S, dtype=np.int32)
        self.T = int(self.S[0].sum())
        ws = max(kvs.kvs_decode_workspace_bytes(c.b, c.Hq, c.Hkv, c.d, row) for row in self.S)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        mb = len(self.parts) if microbatches is None else max(1, min(int(microbatches), c.b))
        self.parts = [(c.b * k // mb, c.b * (k + 1) // mb) for k in range(mb)]
        self.part_ws = [
            torch.empty(max(kvs.kvs_decode_workspace_bytes(r1 - r0, c.Hq, c.Hkv, c.d, row)
                            for row in self.S), dtype=torch.uint8, device=device)
            for r0, r1 in self.parts] if mb > 1 else [self.workspace]

    def queries(self) -> List[torch.Tensor]:
        return [self.wl.q(l, device=self.device) for l in range(self.cfg.L)]

    # ------------------------------------------------------------- per step --
    def select(self, l: int, q: torch.Tensor, stream=None) -> None:
        """Score every page of layer l and keep each head's top-K."""
        c, cache, buf = self.cfg, self.caches[l], self.bufs[l]
        if self.fused[l]:
            kvs.kvs_select_pages(cache, q, buf.scores, c.topk, buf.sel, buf.sel_count, stream)
            return
        kvs.kvs_score_pages(cache, q, buf.scores, stream)
        kvs.kvs_topk_pages(buf.scores, cache.seq_len, c.P, c.topk, buf.sel, buf.sel_count, stream)

    def attend(self, l: int, q: torch.Tensor, stream=None, S_row=None) -> torch.Tensor:
        c, buf = self.cfg, self.bufs[l]
        kvs.kvs_decode_attn(self.caches[l], q, buf.sel, buf.sel_count, c.topk or 0,
                            self.S[l] if S_row is None else S_row, self.scale, self.workspace,
                            buf.out, stream)
        return buf.out

    def run_layer(self, l: int, q: torch.Tensor, stream=None) -> torch.Tensor:
        if self.cfg.topk:
            self.select(l, q, stream)
        return self.attend(l, q, stream)

    def run(self, qs: List[torch.Tensor], stream=None) -> None:
        for l in range(self.cfg.L):
            self.run_layer(l, qs[l], stream)

    def run_part(self, k: int, qs: List[torch.Tensor], stream) -> None:
        """Every layer for the requests of micro-batch k, on ``stream``."""
        c = self.cfg
        r0, r1 = self.parts[k]
        for l in range(c.L):
            cache, buf, q = self.caches[l].rows(r0, r1), self.bufs[l], qs[l][r0:r1]
            if self.fused[l]:
                kvs.kvs_select_pages(cache, q, buf.scores[r0:r1], c.topk, buf.sel[r0:r1],
                                     buf.sel_count[r0:r1], stream)
            elif c.topk:
                kvs.kvs_score_pages(cache, q, buf.scores[r0:r1], stream)
                kvs.kvs_topk_pages(buf.scores[r0:r1], cache.seq_len, c.P, c.topk,
                                   buf.sel[r0:r1], buf.sel_count[r0:r1], stream)
            kvs.kvs_decode_attn(cache, q, buf.sel[r0:r1] if c.topk else None,
                                buf.sel_count[r0:r1] if c.topk else None, c.topk or 0,
                                self.S[l], self.scale, self.part_ws[k], buf.out[r0:r1], stream)

    def capture(self, qs: List[torch.Tensor]) -> "torch.cuda.CUDAGraph":
        """Record one whole step (every layer) as a HIP graph.  Every launch
        has a static grid and takes its arguments by value, and the step
        issues no memset, so a replay re-runs exactly the eager step on the
        buffers bound at capture time.  With several micro-batches the graph
        forks into one stream per part and joins at the end."""
        g = torch.cuda.CUDAGraph()
        if len(self.parts) == 1:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self.run(qs, side)          # warm-up on the capture stream
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                self.run(qs, torch.cuda.current_stream())
            return g
        streams = [torch.cuda.Stream() for _ in self.parts]
        cur = torch.cuda.current_stream()
        for k, s in enumerate(streams):     # warm-up, eagerly, on the same streams
            s.wait_stream(cur)
            self.run_part(k, qs, s)
        for s in streams:
            cur.wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            cur = torch.cuda.current_stream()
            for s in streams:
                s.wait_stream(cur)
            for k, s in enumerate(streams):
                self.run_part(k, qs, s)
            for s in streams:
                cur.wait_stream(s)
        self._graph_streams = streams       # kept alive with the graph
        return g
