"""Chunked prefill under Budget Reservation (Tangram review, 3.1).

Each request's prompt of N tokens arrives in chunks of C.  As a chunk's K/V
is computed, every head keeps its top tokens by a score s; the compressed
footprint is fixed when the request is scheduled -- ceil(B N) tokens per
head -- so pages are reserved up front and nothing is reclaimed later.
Reading used here: the kept count after position x is ceil(B x), so chunk
[a, e) keeps ceil(B e) - ceil(B a) tokens of its own.

The score function belongs to the compression method layered on top (the
pages name several; none is part of this path), so a seeded uniform score
per (token, head) stands in for it.  Everything runs through the C ABI
(``kvs_prefill_chunk``): per chunk and layer, selection, compaction into the
head's ragged pages and the pages' min-max bounds happen in one kernel.
"""

from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np
import torch

from . import kvs
from .pipeline import DecodeStep
from .workloads import Workload, _mix, torch_dtype

__all__ = ["ChunkedPrefill"]


class ChunkedPrefill:
    """Prefill of every layer of a workload, chunk by chunk, into caches whose
    pages are reserved for ceil(B N) tokens per head."""

    def __init__(self, wl: Workload, chunk: int, device="cuda"):
        c = wl.cfg
        if c.nbanks != c.L:
            raise ValueError("prefill needs one physical pool per layer")
        if not 1 <= chunk <= 8192:
            raise ValueError("chunk length must lie in [1, 8192]")
        self.wl, self.cfg, self.device, self.C = wl, c, device, chunk
        whole = int(wl.contexts.max())
        for l in range(c.L):   # the quota of a chunk covering every prompt: ceil(B N)
            if not np.array_equal(kvs.kvs_prefill_quota(wl.budgets[l], wl.contexts, 0, whole),
                                  wl.n[:, l, :]):
                raise ValueError("the reserved length differs from ceil(B N)")
        # the reservation: every head's pages and bounds blocks for n = ceil(B N)
        self.ds = DecodeStep(wl, device=device, poison=True)
        self.chunks = int(-(-int(wl.contexts.max()) // chunk))
        self.workspace = torch.empty(kvs.kvs_prefill_workspace_bytes(c.b, c.Hkv, chunk),
                                     dtype=torch.uint8, device=device)
        self.reset()

    def reset(self) -> None:
        for cache in self.ds.caches:
            cache.seq_len.zero_()

    def quota(self, l: int, k: int) -> np.ndarray:
        """[b][Hkv] tokens each head keeps from chunk k of layer l."""
        return kvs.kvs_prefill_quota(self.wl.budgets[l], self.wl.contexts, k * self.C, self.C)

    def inputs(self, l: int, k: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """Chunk k of layer l: keys and values [b][Hkv][C][d] ~ N(0,1) and
        scores [b][Hkv][C] ~ U[0,1); positions past a request's prompt carry
        -inf, so they are never kept."""
        c = self.cfg
        g = torch.Generator(device=self.device).manual_seed(_mix(c.seed, 7, l, k))
        kv = torch.randn((c.b, c.Hkv, 2, self.C, c.d), generator=g, device=self.device,
                         dtype=torch.float32).to(torch_dtype(c.dtype))
        s = torch.rand((c.b, c.Hkv, self.C), generator=g, device=self.device, dtype=torch.float32)
        for r in range(c.b):
            valid = int(self.wl.contexts[r]) - k * self.C
            if valid < self.C:
                s[r, :, max(0, valid):] = -math.inf
        return kv[:, :, 0].contiguous(), kv[:, :, 1].contiguous(), s

    def run_chunk(self, l: int, k: int, inputs=None, quota=None, stream=None) -> None:
        kc, vc, s = inputs if inputs is not None else self.inputs(l, k)
        q = quota if quota is not None else torch.from_numpy(self.quota(l, k)).to(self.device)
        kvs.kvs_prefill_chunk(self.ds.caches[l], kc, vc, s, q, self.workspace, stream)
