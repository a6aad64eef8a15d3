"""Builds head-ragged paged KV caches on the device (Tangram review, 3.2
Ragged Paging: per-group page tables, each group sized by its longest head;
FlexiCache summary, System engineering: -1 null entries keep the logical
table dense).

Host-side allocator and packer: page tables are built in numpy, token data
is scattered into the pool with torch device copies.  Physical page ids are
handed out in a seeded shuffled order so that the kernels' table walks are
exercised, not bypassed by a contiguous layout.  Unused pool slots are
filled with NaN so that any read of an invalid token shows up in the output.

The min-max cache (FlexiCache summary, Key observations, assumption 2: page
bounds kept on the GPU apart from the KV pages) is ragged per head: each
(request, head) owns a contiguous run of ceil(n/P) blocks starting at
meta_base[r][h], so scoring streams a head's bounds in page order however
its KV pages are scattered.

Layers whose data share a bank (workload layers l and l + data_layers) share
one physical pool: each (request, group) gets as many pages as the largest
of those layers needs, and every layer has its own page table (a prefix of
the same page list), its own seq_len and its own min-max buffer.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np
import torch

from .kvs import Cache
from .workloads import Workload, torch_dtype

__all__ = ["build_caches", "RaggedLayout"]


@dataclass
class RaggedLayout:
    """Host copy of one layer's tables."""
    page_table: np.ndarray   # [b][G][maxpg] int32, -1 null
    meta_base: np.ndarray    # [b][Hkv] int32, first min-max block of each head
    seq_len: np.ndarray      # [b][Hkv] int32
    head_slot: np.ndarray    # [Hkv] int32
    pool: int                # physical pool index


def _nan_fill(t: torch.Tensor) -> None:
    t.view(torch.int16).fill_(0x7E00 if t.dtype == torch.float16 else 0x7FC0)


def build_caches(wl: Workload, head_slot: np.ndarray, device="cuda", poison: bool = True,
                 seed: int = 1234, growth: int = 0) -> Tuple[List[Cache], List[RaggedLayout]]:
    """Allocate and fill the ragged caches of every layer of ``wl``.

    head_slot: [L][Hkv] pool positions (group = pos // Hp, slot = pos % Hp).
    growth: tokens every head may still append; pages and min-max blocks are
    mapped for n + growth tokens up front, so appends never allocate.
    Returns per-layer device caches (min-max buffers allocated, not built)
    and their host layouts.
    """
    c = wl.cfg
    P, Hp, G, d = c.P, c.Hp, c.G, c.d
    dt = torch_dtype(c.dtype)
    nb = c.nbanks
    per_head = c.retain != "prefix" or c.offsets
    if per_head and nb != c.L:
        raise ValueError("per-head data needs one bank per layer")
    hs = np.asarray(head_slot, dtype=np.int64)
    rng = np.random.default_rng(seed)

    # pages each layer needs per (request, group): its longest head
    need = np.zeros((c.L, c.b, G), dtype=np.int64)
    for l in range(c.L):
        for h in range(c.Hkv):
            i = hs[l, h] // Hp
            need[l, :, i] = np.maximum(need[l, :, i], -(-(wl.n[:, l, h] + growth) // P))

    caches: List[Cache] = [None] * c.L
    layouts: List[RaggedLayout] = [None] * c.L
    for lam in range(nb):
        layers = list(range(lam, c.L, nb))
        R = need[layers].max(axis=0)                      # [b][G]
        total = int(R.sum())
        ids = rng.permutation(total).astype(np.int32)
        starts = np.concatenate([[0], np.cumsum(R.reshape(-1))]).astype(np.int64)
        kv = torch.empty((total, Hp, 2, P, d), dtype=dt, device=device)
        if poison:
            _nan_fill(kv)

        def pages(r, i):
            k = r * G + i
            return ids[starts[k]:starts[k + 1]]

        # token data
        if per_head:
            l = layers[0]
            for r in range(c.b):
                for h in range(c.Hkv):
                    pos = int(hs[l, h])
                    K, V = wl.head_kv(r, l, h, pos, device=device)
                    _scatter(kv, pages(r, pos // Hp), pos % Hp, K, V, P)
        else:
            for r in range(c.b):
                for pos in range(c.Hkv):
                    bank = wl.bank(r, lam, pos, device=device)
                    pg = pages(r, pos // Hp)
                    m = min(bank.shape[0], len(pg) * P)
                    _scatter(kv, pg, pos % Hp, bank[:m, 0], bank[:m, 1], P)
                    del bank

        for l in layers:
            maxpg = int(max(1, need[l].max()))
            pt = np.full((c.b, G, maxpg), -1, dtype=np.int32)
            for r in range(c.b):
                for i in range(G):
                    k = int(need[l, r, i])
                    pt[r, i, :k] = pages(r, i)[:k]
            seq = wl.n[:, l, :].astype(np.int32)
            runs = (-(-(wl.n[:, l, :] + growth) // P)).reshape(-1)
            mb = np.concatenate([[0], np.cumsum(runs)[:-1]]).astype(np.int32).reshape(c.b, c.Hkv)
            mm = torch.empty((max(1, int(runs.sum())), d, 2), dtype=dt, device=device)
            if poison:
                _nan_fill(mm)
            caches[l] = Cache(kv=kv, minmax=mm, meta_base=torch.from_numpy(mb).to(device),
                              page_table=torch.from_numpy(pt).to(device),
                              seq_len=torch.from_numpy(np.ascontiguousarray(seq)).to(device),
                              head_slot=torch.from_numpy(hs[l].astype(np.int32)).to(device),
                              Hq=c.Hq)
            layouts[l] = RaggedLayout(page_table=pt, meta_base=mb, seq_len=seq,
                                      head_slot=hs[l].astype(np.int32), pool=lam)
    return caches, layouts


def _scatter(kv: torch.Tensor, page_ids: np.ndarray, slot: int, K: torch.Tensor,
             V: torch.Tensor, P: int) -> None:
    """Write tokens K[t], V[t] to pool page page_ids[t // P], row t % P of ``slot``."""
    n = K.shape[0]
    full = n // P
    idx = torch.as_tensor(np.asarray(page_ids[:full], dtype=np.int64), device=kv.device)
    if full:
        kv[idx, slot, 0] = K[:full * P].reshape(full, P, -1)
        kv[idx, slot, 1] = V[:full * P].reshape(full, P, -1)
    tail = n - full * P
    if tail:
        pid = int(page_ids[full])
        kv[pid, slot, 0, :tail] = K[full * P:]
        kv[pid, slot, 1, :tail] = V[full * P:]


def unpack_head(kv: torch.Tensor, layout: RaggedLayout, r: int, h: int, P: int):
    """Read a head's tokens back through its page table (test helper)."""
    pos = int(layout.head_slot[h])
    i, j = pos // kv.shape[1], pos % kv.shape[1]
    n = int(layout.seq_len[r, h])
    npg = -(-n // P)
    ids = torch.as_tensor(layout.page_table[r, i, :npg].astype(np.int64), device=kv.device)
    K = kv[ids, j, 0].reshape(npg * P, -1)[:n]
    V = kv[ids, j, 1].reshape(npg * P, -1)[:n]
    return K, V
