"""Decode steps over time: append, stability-aware rerank, selection reuse.

FlexiCache summary, Method: every head is either stable or unstable (an
offline classification; here a seeded stand-in, see
``Workload.stable_heads``).  At each decode step the token being decoded is
appended to the cache first (its page's min-max bounds updated in place),
then unstable heads re-select their top-K pages, stable heads re-select only
every ``period`` steps and otherwise keep the pages of their last rerank,
and a layer whose heads all keep their pages is not scored at all.  The
decode then attends each head's current selection with the tokens its pages
now hold.

Everything runs through the C ABI: ``kvs_append_kv``, then
``kvs_score_pages[_heads]`` and ``kvs_topk_pages[_heads]`` for the heads
that re-select, then ``kvs_decode_attn``.  Pages and min-max blocks for the
appended tokens are mapped when the caches are built (``growth``), so no
step allocates.
"""

from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import kvs
from .pipeline import DecodeStep
from .workloads import Workload

__all__ = ["DecodeLoop", "heads_due"]


def heads_due(t: int, stable: np.ndarray, period: int) -> np.ndarray:
    """KV heads that re-select their pages at step t (counted from the first
    decode step): every head on a rerank step (t a multiple of the period),
    otherwise the unstable ones (kvs_rerank_heads)."""
    return kvs.kvs_rerank_heads(stable, t, period)


class DecodeLoop:
    def __init__(self, wl: Workload, steps: int, device="cuda", period: int = 16,
                 unstable_frac: float = 0.25, T: Optional[int] = None, poison: bool = True,
                 stable: Optional[np.ndarray] = None):
        c = wl.cfg
        if not c.topk:
            raise ValueError("the rerank schedule needs a top-K workload")
        if c.nbanks != c.L:
            raise ValueError("appends need one physical pool per layer (aliased pools would "
                             "overwrite another layer's tokens)")
        if period < 1 or steps < 1:
            raise ValueError("steps >= 1 and period >= 1 required")
        self.wl, self.cfg, self.device = wl, c, device
        self.steps, self.period = steps, period
        self.ds = DecodeStep(wl, device=device, T=T, poison=poison, growth=steps)
        self.stable = (wl.stable_heads(unstable_frac) if stable is None
                       else np.array(stable, dtype=bool))       # [L][Hkv]
        self.n0 = [cache.seq_len.clone() for cache in self.ds.caches]
        # the bounds as built: an append merges its token into its page's
        # bounds, so a rewind has to restore them as well as the lengths
        self.mm0 = [cache.minmax.clone() for cache in self.ds.caches]
        # every step's inputs, resident on the device before any step runs
        qs = [wl.step_qs(steps, l, device) for l in range(c.L)]
        self.q = [[qs[l][t] for l in range(c.L)] for t in range(steps)]
        self.kv = [[wl.step_kv(t, l, device) for l in range(c.L)] for t in range(steps)]

    def heads_due(self, t: int, l: int) -> np.ndarray:
        return heads_due(t, self.stable[l], self.period)

    def rewind(self) -> None:
        """Back to the state before step 0: the tokens each head held when the
        caches were built and the bounds of their pages.  Re-running the same
        steps rewrites the same tokens, so every step of a rewound replay sees
        exactly the state the same step saw the first time."""
        for cache, n0, mm0 in zip(self.ds.caches, self.n0, self.mm0):
            cache.seq_len.copy_(n0)
            cache.minmax.copy_(mm0)

    def run_layer(self, t: int, l: int, stream=None, reuse: bool = True) -> torch.Tensor:
        c, ds = self.cfg, self.ds
        cache, buf = ds.caches[l], ds.bufs[l]
        k, v = self.kv[t][l]
        kvs.kvs_append_kv(cache, k, v, stream)
        due = self.heads_due(t, l) if reuse else np.ones(c.Hkv, dtype=bool)
        if due.all():
            ds.select(l, self.q[t][l], stream)
        elif due.any():
            kvs.kvs_score_pages(cache, self.q[t][l], buf.scores, stream, heads=due)
            kvs.kvs_topk_pages(buf.scores, cache.seq_len, c.P, c.topk, buf.sel, buf.sel_count,
                               stream, heads=due)
        return ds.attend(l, self.q[t][l], stream)

    def run_step(self, t: int, stream=None, reuse: bool = True) -> None:
        for l in range(self.cfg.L):
            self.run_layer(t, l, stream, reuse)

    def capture(self, t1: int, reuse: bool = True) -> "torch.cuda.CUDAGraph":
        """Steps [0, t1) as one HIP graph (every step's inputs are distinct
        device tensors, so one graph holds the whole window).  A replay runs
        those steps from whatever state the caches are in: ``rewind`` before
        each replay to repeat them from the start.  Leaves the caches
        rewound."""
        if not 1 <= t1 <= self.steps:
            raise ValueError("window must lie within the prepared steps")
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        self.rewind()
        with torch.cuda.stream(side):
            for t in range(t1):                # warm-up on the capture stream
                self.run_step(t, side, reuse)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.rewind()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for t in range(t1):
                self.run_step(t, torch.cuda.current_stream(), reuse)
        torch.cuda.synchronize()
        self.rewind()
        torch.cuda.synchronize()
        return g

    def outputs(self) -> List[torch.Tensor]:
        return [b.out for b in self.ds.bufs]
