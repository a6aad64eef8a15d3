"""Tiered placement of stable heads (FlexiCache summary, tiered placement).

Unstable heads keep every page on the GPU.  A stable head keeps only the
pages of its current top-K selection on the GPU, in ``slots`` GPU pages it
owns; all of its pages live in pinned host memory, and a rerank moves only
the pages newly promoted into the selection (``kvs_promote_pages``: the
freed slots are reused in the same kernel, the copies read host memory
directly).  The min-max bounds of every page stay on the GPU, so scoring
never waits on the host tier; a page held only on the host has the table
entry KVS_PAGE_ON_HOST, which scoring treats as present and the decode as
absent.

Set-up follows the pages' order: the full cache is built on the GPU (the
stand-in for prefill) with its bounds, the stable heads' pages are offloaded
in bulk (``kvs_offload_pages``), then the GPU pool is compacted to the
unstable heads' pages plus the stable heads' slots -- a host-side
re-layout, like the rest of the allocator in layout.py.

Each step runs the rerank schedule of ``steps.heads_due``: the heads due
re-select, and the tiered ones among them promote.  With ``append=True`` the
step first appends its token, written through to the tiered heads' host
pages (``kvs_append_kv_tier``), so the host copy of every page, newly filled
ones included, stays complete.  The same schedule on the fully resident
cache gives the same selections and, because the decode reads only selected
pages, the same outputs bit for bit.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import kvs
from .kvs import KVS_PAGE_ON_HOST, Cache, Tier
from .pipeline import DecodeStep
from .steps import heads_due
from .workloads import Workload, torch_dtype

__all__ = ["TieredLoop", "build_tier", "TierLayout"]


@dataclass
class TierLayout:
    """Host copy of one layer's tier tables."""
    host_base: np.ndarray    # [b][Hkv] int64, -1: not tiered
    slot_phys: np.ndarray    # [b][Hkv][slots] int32
    page_table: np.ndarray   # [b][Hkv][maxpg] int32 after compaction
    gpu_pages: int           # pages in the compacted GPU pool
    full_pages: int          # pages of the fully resident pool


def build_tier(cache: Cache, stable: np.ndarray, slots: int, seed: int = 99):
    """Offload the stable heads of ``cache`` (a fully resident cache with one
    head per page table) to pinned host memory and compact its GPU pool.

    stable: [Hkv] bool, the heads to tier (in every request).
    Returns (tiered cache, Tier, TierLayout); the old pool is no longer
    referenced by the result.
    """
    num_pages, Hp, two, P, d = cache.kv.shape
    if Hp != 1:
        raise ValueError("a host tier needs one head per page table (Hp == 1)")
    dev, dt = cache.kv.device, cache.kv.dtype
    b, Hkv = cache.seq_len.shape
    maxpg = cache.page_table.shape[2]
    pt = cache.page_table.cpu().numpy()
    hs = cache.head_slot.cpu().numpy()
    tiered = np.broadcast_to(np.asarray(stable, dtype=bool)[None, :], (b, Hkv))

    # every mapped page of a tiered head gets a host page, the pages mapped
    # for tokens still to be appended included
    mapped = np.zeros((b, Hkv), dtype=np.int64)
    for r in range(b):
        for h in range(Hkv):
            got = np.nonzero(pt[r, hs[h]] >= 0)[0]
            mapped[r, h] = int(got[-1]) + 1 if got.size else 0
    host_base = np.full((b, Hkv), -1, dtype=np.int64)
    run = 0
    for r in range(b):
        for h in range(Hkv):
            if tiered[r, h]:
                host_base[r, h] = run
                run += int(mapped[r, h])
    host_kv = torch.empty((max(1, run), 2, P, d), dtype=dt, pin_memory=True)
    hb_dev = torch.from_numpy(host_base).to(dev)
    scratch = torch.full((b, Hkv, slots), -1, dtype=torch.int32, device=dev)
    kvs.kvs_offload_pages(cache, Tier(host_kv, hb_dev, scratch, scratch), None)
    torch.cuda.synchronize(dev)

    # compacted pool: the untiered heads' resident pages, then every tiered
    # head's slots, at seeded shuffled physical ids
    keep_old, owners = [], []
    for r in range(b):
        for h in range(Hkv):
            if not tiered[r, h]:
                row = pt[r, hs[h]]
                for p in range(maxpg):
                    if row[p] >= 0:
                        keep_old.append(int(row[p]))
                        owners.append((r, h, p))
    n_slots = int(tiered.sum()) * slots
    total = len(keep_old) + n_slots
    ids = np.random.default_rng(seed).permutation(total).astype(np.int32)
    new_pt = np.full((b, Hkv, maxpg), -1, dtype=np.int32)
    for (r, h, p), nid in zip(owners, ids[:len(keep_old)]):
        new_pt[r, hs[h], p] = nid
    slot_phys = np.full((b, Hkv, slots), -1, dtype=np.int32)
    k = len(keep_old)
    for r in range(b):
        for h in range(Hkv):
            if tiered[r, h]:
                slot_phys[r, h] = ids[k:k + slots]
                k += slots
                row = pt[r, hs[h]]
                m = int(mapped[r, h])
                new_pt[r, hs[h], :m][row[:m] >= 0] = KVS_PAGE_ON_HOST

    kv = torch.empty((max(1, total), 1, 2, P, d), dtype=dt, device=dev)
    kv.view(torch.int16).fill_(0x7E00 if dt == torch.float16 else 0x7FC0)   # NaN: unread slots
    if keep_old:
        src = torch.as_tensor(np.asarray(keep_old, dtype=np.int64), device=dev)
        dst = torch.as_tensor(ids[:len(keep_old)].astype(np.int64), device=dev)
        kv.index_copy_(0, dst, cache.kv.index_select(0, src))
    new = Cache(kv=kv, minmax=cache.minmax, meta_base=cache.meta_base,
                page_table=torch.from_numpy(new_pt).to(dev), seq_len=cache.seq_len,
                head_slot=cache.head_slot, Hq=cache.Hq)
    tier = Tier(host_kv, hb_dev, torch.full((b, Hkv, slots), -1, dtype=torch.int32, device=dev),
                torch.from_numpy(slot_phys).to(dev))
    return new, tier, TierLayout(host_base, slot_phys, new_pt, total, num_pages)


class TieredLoop:
    """Decode steps over a fixed cache under the rerank schedule, with the
    stable heads' pages in a host tier (``tiered=True``) or all on the GPU
    (``tiered=False``, the same schedule without promotion)."""

    def __init__(self, wl: Workload, steps: int, device="cuda", period: int = 16,
                 unstable_frac: float = 0.25, slots: Optional[int] = None, tiered: bool = True,
                 T: Optional[int] = None, stable: Optional[np.ndarray] = None,
                 append: bool = False):
        c = wl.cfg
        if not c.topk:
            raise ValueError("tiered placement needs a top-K workload")
        if c.Hp != 1:
            raise ValueError("tiered placement needs one head per page table (Hp == 1)")
        if c.nbanks != c.L:
            raise ValueError("tiered placement needs one physical pool per layer")
        if period < 1 or steps < 1:
            raise ValueError("steps >= 1 and period >= 1 required")
        self.wl, self.cfg, self.device = wl, c, device
        self.steps, self.period, self.tiered, self.append = steps, period, tiered, append
        self.slots = c.topk if slots is None else int(slots)
        self.ds = DecodeStep(wl, device=device, T=T, poison=True, growth=steps if append else 0)
        self.stable = (wl.stable_heads(unstable_frac) if stable is None
                       else np.asarray(stable, dtype=bool))            # [L][Hkv]
        self.full_bytes = sum(cc.kv.numel() * cc.kv.element_size() for cc in self.ds.caches)
        self.tiers: List[Optional[Tier]] = [None] * c.L
        self.tier_layouts: List[Optional[TierLayout]] = [None] * c.L
        if tiered:
            for l in range(c.L):
                cache, tier, lay = build_tier(self.ds.caches[l], self.stable[l], self.slots,
                                              seed=c.seed + 17 * l)
                self.ds.caches[l], self.tiers[l], self.tier_layouts[l] = cache, tier, lay
            torch.cuda.synchronize()
        self.gpu_bytes = sum(cc.kv.numel() * cc.kv.element_size() for cc in self.ds.caches)
        self.pt0 = [cc.page_table.clone() for cc in self.ds.caches]
        self.n0 = [cc.seq_len.clone() for cc in self.ds.caches]
        self.mm0 = [cc.minmax.clone() for cc in self.ds.caches] if append else None
        self.moved = [torch.zeros((c.b, c.Hkv), dtype=torch.int32, device=device)
                      for _ in range(c.L)]
        qs = [wl.step_qs(steps, l, device) for l in range(c.L)]
        self.q = [[qs[l][t] for l in range(c.L)] for t in range(steps)]
        self.kv = ([[wl.step_kv(t, l, device) for l in range(c.L)] for t in range(steps)]
                   if append else None)

    def heads_due(self, t: int, l: int) -> np.ndarray:
        return heads_due(t, self.stable[l], self.period)

    def select(self, t: int, l: int, stream=None) -> np.ndarray:
        """Re-select the heads due at step t; returns that mask."""
        c, ds = self.cfg, self.ds
        cache, buf = ds.caches[l], ds.bufs[l]
        due = self.heads_due(t, l)
        if due.all():
            ds.select(l, self.q[t][l], stream)
        elif due.any():
            kvs.kvs_score_pages(cache, self.q[t][l], buf.scores, stream, heads=due)
            kvs.kvs_topk_pages(buf.scores, cache.seq_len, c.P, c.topk, buf.sel, buf.sel_count,
                               stream, heads=due)
        return due

    def promote(self, l: int, due: np.ndarray, stream=None) -> None:
        """Make the new selections of the tiered heads among ``due`` resident."""
        if self.tiered and (due & self.stable[l]).any():
            buf = self.ds.bufs[l]
            kvs.kvs_promote_pages(self.ds.caches[l], self.tiers[l], buf.sel, buf.sel_count,
                                  self.cfg.topk, heads=due & self.stable[l],
                                  moved=self.moved[l], stream=stream)

    def run_layer(self, t: int, l: int, stream=None) -> torch.Tensor:
        if self.append:
            k, v = self.kv[t][l]
            if self.tiered:
                kvs.kvs_append_kv_tier(self.ds.caches[l], self.tiers[l], k, v, stream)
            else:
                kvs.kvs_append_kv(self.ds.caches[l], k, v, stream)
        due = self.select(t, l, stream)
        self.promote(l, due, stream)
        return self.ds.attend(l, self.q[t][l], stream)

    def run_step(self, t: int, stream=None) -> None:
        for l in range(self.cfg.L):
            self.run_layer(t, l, stream)

    def rewind(self) -> None:
        """Back to the state before step 0: no stable-head page resident and,
        with appends, the tokens each head held when the caches were built and
        the bounds of their pages (re-running the steps rewrites the same
        rows)."""
        for l in range(self.cfg.L):
            self.ds.caches[l].page_table.copy_(self.pt0[l])
            self.ds.caches[l].seq_len.copy_(self.n0[l])
            if self.mm0 is not None:
                self.ds.caches[l].minmax.copy_(self.mm0[l])
            if self.tiers[l] is not None:
                self.tiers[l].slot_page.fill_(-1)

    def capture(self, t1: int) -> "torch.cuda.CUDAGraph":
        """Steps [0, t1) as one HIP graph; a replay runs them from whatever
        state the tier is in (``rewind`` first to repeat them from the
        start).  Leaves the tier rewound."""
        if not 1 <= t1 <= self.steps:
            raise ValueError("window must lie within the prepared steps")
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        self.rewind()
        with torch.cuda.stream(side):
            for t in range(t1):                # warm-up on the capture stream
                self.run_step(t, side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.rewind()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for t in range(t1):
                self.run_step(t, torch.cuda.current_stream())
        torch.cuda.synchronize()
        self.rewind()
        torch.cuda.synchronize()
        return g

    def outputs(self) -> List[torch.Tensor]:
        return [b.out for b in self.ds.bufs]
