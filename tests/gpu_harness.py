"""Shared GPU-vs-oracle parity checks (test infrastructure).

The oracle side gets each head's tokens straight from the seeded generator
(never through the device pool or page tables) and recomputes everything in
fp64.  The GPU side runs the library through the Python binding.
"""

from __future__ import annotations

import math
import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle as O
from non_uniform_sparse_amd.pipeline import DecodeStep

# Tolerances.  Scores: fp32 sums of exact products, error <= ~1e-6 of the
# absolute term sum A_p.  Selection: set-exact outside a band of 1e-6
# relative around the K-th score.  Attention output (fp16/bf16 KV, fp32
# accumulation): max-abs 1e-2 and relative L2 5e-3.
SCORE_TOL = 1e-6
BAND = 1e-6
OUT_MAX_ABS = 1e-2
OUT_REL_L2 = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU test needs a ROCm device"


def oracle_slots(wl) -> np.ndarray:
    c = wl.cfg
    if c.clustered:
        return np.stack([O.cluster_heads(wl.budgets[l], c.Hp) for l in range(c.L)])
    return np.tile(np.arange(c.Hkv), (c.L, 1))


def head64(wl, r, l, h, pos, device):
    K, V = wl.head_kv(r, l, h, int(pos), device=device)
    return K.double().cpu().numpy(), V.double().cpu().numpy()


@dataclass
class Stats:
    minmax_checked: int = 0
    scores_checked: int = 0
    score_err_max: float = 0.0
    topk_heads: int = 0
    band_events: List[tuple] = field(default_factory=list)
    out_max_abs: float = 0.0
    out_sq_err: float = 0.0
    out_sq_ref: float = 0.0
    out_rows: int = 0

    @property
    def rel_l2(self) -> float:
        return math.sqrt(self.out_sq_err / max(self.out_sq_ref, 1e-300))


def check_layer(step: DecodeStep, l: int, q: torch.Tensor, requests: Sequence[int],
                stats: Stats, check_minmax: bool = True, S_row=None) -> None:
    """Runs layer l on the GPU and checks every step of it against the oracle
    for the given requests (all heads)."""
    wl, c = step.wl, step.cfg
    dev = step.device
    slots = oracle_slots(wl)
    assert np.array_equal(slots[l], step.head_slot[l]), "clustering differs from the oracle"
    cache, lay = step.caches[l], step.layouts[l]
    if S_row is None:
        out = step.run_layer(l, q)          # the path the step takes for this layer
    else:
        if c.topk:
            step.select(l, q)
        out = step.attend(l, q, S_row=S_row)
    torch.cuda.synchronize()
    q64 = q.double().cpu().numpy()
    out_h = out.cpu().numpy().astype(np.float64)
    mm = cache.minmax
    buf = step.bufs[l]
    if c.topk:
        scores = buf.scores.cpu().numpy()
        sel = buf.sel.cpu().numpy()
        cnt = buf.sel_count.cpu().numpy()
    scale = 1.0 / math.sqrt(c.d)
    for r in requests:
        for h in range(c.Hkv):
            pos = int(slots[l, h])
            gi, j = pos // c.Hp, pos % c.Hp
            n = int(wl.n[r, l, h])
            npg = -(-n // c.P)
            K64, V64 = head64(wl, r, l, h, pos, dev)
            assert K64.shape[0] == n
            lo, hi = O.page_minmax(K64, c.P)
            if check_minmax or c.topk:
                m0 = int(lay.meta_base[r, h])
                g_mm = mm[m0:m0 + npg].double().cpu().numpy()     # [npg][d][2]
                if check_minmax:
                    assert np.array_equal(g_mm[:, :, 0], lo), f"kmin r={r} l={l} h={h}"
                    assert np.array_equal(g_mm[:, :, 1], hi), f"kmax r={r} l={l} h={h}"
                    stats.minmax_checked += npg
            qg = q64[r, h * c.Gq:(h + 1) * c.Gq]
            if c.topk:
                s_ora = O.page_scores(qg, lo, hi)
                A = np.max(np.abs(qg[:, None, :] * lo[None]).sum(-1) +
                           np.abs(qg[:, None, :] * hi[None]).sum(-1), axis=0)
                s_gpu = scores[r, h, :npg].astype(np.float64)
                err = np.abs(s_gpu - s_ora) / A
                e_max = float(err.max()) if npg else 0.0     # a head with no token has no page
                assert e_max <= SCORE_TOL, f"score r={r} l={l} h={h} err={e_max}"
                assert np.all(np.isneginf(scores[r, h, npg:]))
                stats.score_err_max = max(stats.score_err_max, e_max)
                stats.scores_checked += npg
                # top-K: exact on the GPU's own fp32 scores ...
                keep = min(c.topk, npg)
                assert cnt[r, h] == keep
                got = sel[r, h, :keep]
                want = O.topk_pages(scores[r, h, :npg], c.topk)
                assert np.array_equal(got, want), f"topk r={r} l={l} h={h}"
                assert np.all(sel[r, h, keep:] == -1)
                # ... and against the oracle's scores decided in fp32, up to near-ties
                ref = O.topk_pages(s_ora.astype(np.float32), c.topk)
                if not np.array_equal(got, ref):
                    tau = float(np.sort(s_ora)[::-1][keep - 1])
                    for p in set(got.tolist()) ^ set(ref.tolist()):
                        assert abs(s_ora[p] - tau) <= BAND * abs(tau), \
                            f"out-of-band selection difference r={r} l={l} h={h} p={p}"
                        stats.band_events.append((c.name, r, l, h, p, float(s_ora[p]), tau))
                stats.topk_heads += 1
                pages = got
            else:
                pages = np.arange(npg)
            ref_o = O.decode_head(qg, K64, V64, pages, c.P, scale)
            g_o = out_h[r, h * c.Gq:(h + 1) * c.Gq]
            assert np.all(np.isfinite(g_o)), f"non-finite output r={r} l={l} h={h}"
            stats.out_max_abs = max(stats.out_max_abs, float(np.abs(g_o - ref_o).max()))
            stats.out_sq_err += float(((g_o - ref_o) ** 2).sum())
            stats.out_sq_ref += float((ref_o ** 2).sum())
            stats.out_rows += c.Gq


def assert_output_bar(stats: Stats, label: str) -> None:
    say(f"{label}: minmax pages {stats.minmax_checked}, scores {stats.scores_checked} "
        f"(max err/A {stats.score_err_max:.2e}), topk heads {stats.topk_heads}, "
        f"band events {len(stats.band_events)}, out rows {stats.out_rows} "
        f"max-abs {stats.out_max_abs:.2e} rel-L2 {stats.rel_l2:.2e}")
    assert stats.out_max_abs <= OUT_MAX_ABS, stats.out_max_abs
    assert stats.rel_l2 <= OUT_REL_L2, stats.rel_l2
