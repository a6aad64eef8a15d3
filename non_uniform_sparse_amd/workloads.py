"""Seeded synthetic inputs for the decode path (shared by tests and bench).

This module only draws random inputs in the shapes, sizes and distributions
of the five workloads below.  It holds none of the decode path's arithmetic
(no min-max, score, selection, planning or attention) and imports nothing
from the HIP binding or from the oracle.

Workloads (all seed 0, page size 16):
  tiny_ragged      1 request, 1 layer, 32q/8kv, d=128, fp16, context 4096,
                   budgets U[0.1,1]; each head keeps ceil(B*4096) tokens chosen
                   by a random score, in position order; dense over them.
  llama8b_ragged   16 requests, 1 layer, 32q/8kv, d=128, fp16, context 32768,
                   budgets min(1, 2*x*0.3/mean(x)), x ~ Beta(2,5) per head.
  flexicache_topk  40 requests, 1 layer, 32q/8kv, d=128, fp16, 10240 tokens
                   (640 pages) per head all kept; 5% of each head's pages get
                   +3 on 8 random channels of K; top-64 pages per KV head.
  longctx_skew     4 requests, 32 layers, 32q/8kv, d=128, bf16, 100000 tokens;
                   26 of 256 (layer, head) budgets at 1.0, the rest
                   clip(LogNormal(-2.2, 0.6), 0.02, 1).
  gemma3_mixed     64 requests, 48 layers, 16q/8kv, d=256, bf16, contexts
                   round(exp(N(ln(2048*sqrt(32)), ln(32)/6))) clipped to
                   [2048, 65536]; budgets min(1, x*0.5/mean(x)), x ~ Beta(2,5)
                   per (layer, head); top-128 pages per KV head.  Layers share
                   8 data banks (layer l reads bank l mod 8) so the ragged
                   caches of all 48 layers fit one GPU.

Data model.  Host draws (budgets, retention picks, contexts, offsets) come
from one numpy PCG64(seed) stream in that order.  Token data come from
"banks": bank (r, lam, pos) holds bank_len(r, lam) tokens of K and V ~ N(0,1),
drawn by a torch generator seeded from (seed, r, lam, pos).  Head h of layer
l of request r stored at pool position pos reads the first n[r,l,h] tokens
of bank (r, l mod data_layers, pos).  The tiny workload instead draws a full
4096-token stream per head and keeps the chosen positions.

Decoding over steps.  The token appended at step t is N(0,1).  The query
drifts from step to step: an AR(1) process with per-step correlation
QUERY_RHO (``step_qs``), so that top-K sets turn over between reranks at
the rate the pages report.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

__all__ = ["Config", "CONFIGS", "Workload", "make_workload", "torch_dtype"]


@dataclass(frozen=True)
class Config:
    name: str
    b: int
    L: int
    Hq: int
    Hkv: int
    d: int
    dtype: str                 # "f16" or "bf16"
    N: int                     # context per request (max for lognormal contexts)
    budget: str                # budget recipe
    clustered: bool            # heads grouped by budget (else identity grouping)
    topk: Optional[int] = None  # pages per KV head, None = attend every retained page
    P: int = 16
    Hp: int = 4
    data_layers: Optional[int] = None   # banks shared across layers (None = one per layer)
    contexts: str = "fixed"    # "fixed" or "lognormal"
    retain: str = "prefix"     # "prefix" (iid tokens) or "random_score"
    offsets: bool = False      # +3 key offsets on 5% of pages, 8 random channels
    seed: int = 0

    @property
    def Gq(self) -> int:
        return self.Hq // self.Hkv

    @property
    def G(self) -> int:
        return self.Hkv // self.Hp

    @property
    def nbanks(self) -> int:
        return min(self.data_layers, self.L) if self.data_layers else self.L


CONFIGS: Dict[str, Config] = {
    "tiny_ragged": Config("tiny_ragged", b=1, L=1, Hq=32, Hkv=8, d=128, dtype="f16", N=4096,
                          budget="uniform", clustered=False, retain="random_score"),
    "llama8b_ragged": Config("llama8b_ragged", b=16, L=1, Hq=32, Hkv=8, d=128, dtype="f16",
                             N=32768, budget="beta_alpha", clustered=True),
    "flexicache_topk": Config("flexicache_topk", b=40, L=1, Hq=32, Hkv=8, d=128, dtype="f16",
                              N=10240, budget="full", clustered=True, topk=64, offsets=True),
    "longctx_skew": Config("longctx_skew", b=4, L=32, Hq=32, Hkv=8, d=128, dtype="bf16",
                           N=100000, budget="heavy_tail", clustered=True),
    "gemma3_mixed": Config("gemma3_mixed", b=64, L=48, Hq=16, Hkv=8, d=256, dtype="bf16",
                           N=65536, budget="beta_mean", clustered=True, topk=128,
                           data_layers=8, contexts="lognormal"),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f16": torch.float16, "bf16": torch.bfloat16}[name]


# Step-to-step correlation of decode queries (see Workload.step_qs).
QUERY_RHO = 0.997


def _mix(*vals: int) -> int:
    """Deterministic 63-bit seed from a tuple of small integers (splitmix64 steps)."""
    x = 0x9E3779B97F4A7C15
    mask = (1 << 64) - 1
    for v in vals:
        x = (x ^ (int(v) & mask)) & mask
        x = (x + 0x9E3779B97F4A7C15) & mask
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        x = z ^ (z >> 31)
    return x & ((1 << 63) - 1)


def _draw_budgets(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    L, H = cfg.L, cfg.Hkv
    if cfg.budget == "uniform":
        return rng.uniform(0.1, 1.0, (L, H))
    if cfg.budget == "full":
        return np.ones((L, H))
    if cfg.budget == "beta_alpha":           # alpha = 2, rho = 0.3, same for every request
        x = rng.beta(2.0, 5.0, (L, H))
        return np.minimum(1.0, 2.0 * x * 0.3 / x.mean())
    if cfg.budget == "beta_mean":            # rho = 0.5, no safety factor
        x = rng.beta(2.0, 5.0, (L, H))
        return np.minimum(1.0, x * 0.5 / x.mean())
    if cfg.budget == "heavy_tail":           # 10% of (layer, head) at 1.0
        total = L * H
        ones = int(round(0.1 * total))
        B = np.clip(rng.lognormal(-2.2, 0.6, total), 0.02, 1.0)
        B[rng.permutation(total)[:ones]] = 1.0
        return B.reshape(L, H)
    raise ValueError(cfg.budget)


@dataclass
class Workload:
    cfg: Config
    budgets: np.ndarray            # [L][Hkv] float64
    contexts: np.ndarray           # [b] int64
    n: np.ndarray                  # [b][L][Hkv] int64 retained tokens
    retained_pos: Dict[Tuple[int, int, int], np.ndarray] = field(default_factory=dict)
    offsets: Dict[Tuple[int, int], list] = field(default_factory=dict)  # (r, h) -> [(page, channels)]

    # ----------------------------------------------------------------- sizes --
    def bank_len(self, r: int, lam: int) -> int:
        ls = range(lam, self.cfg.L, self.cfg.nbanks)
        return int(max(self.n[r, l].max() for l in ls))

    def q(self, l: int, device="cpu") -> torch.Tensor:
        """Decode queries of layer l: [b][Hq][d] ~ N(0,1) in the workload dtype."""
        c = self.cfg
        g = torch.Generator(device=device).manual_seed(_mix(c.seed, 1, l))
        x = torch.randn((c.b, c.Hq, c.d), generator=g, device=device, dtype=torch.float32)
        return x.to(torch_dtype(c.dtype))

    def bank(self, r: int, lam: int, pos: int, device="cpu") -> torch.Tensor:
        """Bank tokens [bank_len][2][d] (index 0 = K, 1 = V), N(0,1)."""
        c = self.cfg
        g = torch.Generator(device=device).manual_seed(_mix(c.seed, 2, r, lam, pos))
        x = torch.randn((self.bank_len(r, lam), 2, c.d), generator=g, device=device,
                        dtype=torch.float32)
        return x.to(torch_dtype(c.dtype))

    def head_kv(self, r: int, l: int, h: int, pos: int, device="cpu",
                bank: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
        """Retained keys and values [n][d] of head h (layer l, request r) that
        sits at pool position pos.  ``bank`` may pass the already drawn bank."""
        c = self.cfg
        n = int(self.n[r, l, h])
        if c.retain == "random_score":
            g = torch.Generator(device=device).manual_seed(_mix(c.seed, 3, r, l, h))
            full = torch.randn((c.N, 2, c.d), generator=g, device=device, dtype=torch.float32)
            idx = torch.as_tensor(self.retained_pos[(r, l, h)], device=device)
            kv = full[idx].to(torch_dtype(c.dtype))
        else:
            if bank is None:
                bank = self.bank(r, l % c.nbanks, pos, device)
            kv = bank[:n]
        K = kv[:, 0].clone()
        V = kv[:, 1].clone()
        if c.offsets:
            for page, chans in self.offsets.get((r, h), ()):
                lo, hi = page * c.P, min(n, (page + 1) * c.P)
                if lo < hi:
                    ch = torch.as_tensor(chans, device=device)
                    K[lo:hi, ch] = (K[lo:hi, ch].float() + 3.0).to(K.dtype)
        return K, V

    # ---------------------------------------------------------- decode steps --
    def step_qs(self, steps: int, l: int, device="cpu") -> List[torch.Tensor]:
        """Queries of decode steps 0 .. steps-1 of layer l, each [b][Hq][d].

        A query drifts from step to step rather than being drawn afresh: an
        AR(1) process q_t = rho q_{t-1} + sqrt(1 - rho^2) e_t with q_0 = e_0
        and e_t ~ N(0,1) (every q_t is N(0,1) too).  rho = QUERY_RHO is set
        so that the top-K set of a flexicache_topk head re-selected every 16
        steps changes by about 30% (simulated: 31%), inside the 23-35% of
        promoted pages per rerank that the FlexiCache summary (tiered
        placement) reports for real attention.  Computed in fp32, then cast
        to the workload dtype."""
        c = self.cfg
        out, q = [], None
        a = math.sqrt(1.0 - QUERY_RHO * QUERY_RHO)
        for t in range(steps):
            g = torch.Generator(device=device).manual_seed(_mix(c.seed, 4, t, l))
            e = torch.randn((c.b, c.Hq, c.d), generator=g, device=device, dtype=torch.float32)
            q = e if q is None else QUERY_RHO * q + a * e
            out.append(q.to(torch_dtype(c.dtype)))
        return out

    def step_q(self, t: int, l: int, device="cpu") -> torch.Tensor:
        """Queries of decode step t of layer l (see ``step_qs``)."""
        return self.step_qs(t + 1, l, device)[t]

    def step_kv(self, t: int, l: int, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
        """Key and value of the token decoded at step t, for every (request,
        KV head) of layer l: two [b][Hkv][d] tensors ~ N(0,1)."""
        c = self.cfg
        g = torch.Generator(device=device).manual_seed(_mix(c.seed, 5, t, l))
        x = torch.randn((c.b, c.Hkv, 2, c.d), generator=g, device=device, dtype=torch.float32)
        x = x.to(torch_dtype(c.dtype))
        return x[:, :, 0].contiguous(), x[:, :, 1].contiguous()

    def stable_heads(self, unstable_frac: float = 0.25) -> np.ndarray:
        """[L][Hkv] bool, False for the heads treated as unstable.  Stands in
        for the offline head classification (the least temporally stable
        quarter of all heads, FlexiCache summary, Method), which needs real
        attention data: a seeded choice of round(frac * L * Hkv) of all
        (layer, head) pairs, so some layers have no unstable head."""
        c = self.cfg
        total = c.L * c.Hkv
        rng = np.random.default_rng(_mix(c.seed, 6))
        flags = np.ones(total, dtype=bool)
        flags[rng.permutation(total)[:int(round(unstable_frac * total))]] = False
        return flags.reshape(c.L, c.Hkv)


def make_workload(name: str, **overrides) -> Workload:
    """Draw the host-side structure of a workload.  ``overrides`` may shrink
    it (e.g. b, L, N) for quick tests; the recipe is otherwise unchanged."""
    cfg = replace(CONFIGS[name], **overrides)
    rng = np.random.default_rng(cfg.seed)
    budgets = _draw_budgets(cfg, rng)
    # retained token counts, ceil(B * N) per (request, layer, head)
    retained_pos = {}
    if cfg.retain == "random_score":
        contexts = np.full(cfg.b, cfg.N, dtype=np.int64)
        n = np.empty((cfg.b, cfg.L, cfg.Hkv), dtype=np.int64)
        for r in range(cfg.b):
            for l in range(cfg.L):
                for h in range(cfg.Hkv):
                    cnt = int(math.ceil(budgets[l, h] * cfg.N))
                    score = rng.random(cfg.N)
                    # keep the cnt highest scores, equal scores by lower position
                    order = np.lexsort((np.arange(cfg.N), -score))[:cnt]
                    retained_pos[(r, l, h)] = np.sort(order)
                    n[r, l, h] = cnt
    else:
        if cfg.contexts == "lognormal":
            mu, sigma = math.log(2048 * math.sqrt(32)), math.log(32) / 6
            contexts = np.clip(np.rint(rng.lognormal(mu, sigma, cfg.b)), 2048, cfg.N).astype(np.int64)
        else:
            contexts = np.full(cfg.b, cfg.N, dtype=np.int64)
        n = np.ceil(budgets[None, :, :] * contexts[:, None, None]).astype(np.int64)
    n = np.maximum(n, 1)
    offsets = {}
    if cfg.offsets:
        for r in range(cfg.b):
            for h in range(cfg.Hkv):
                npg = -(-int(n[r, 0, h]) // cfg.P)
                k = max(1, int(round(0.05 * npg)))
                pages = rng.choice(npg, size=k, replace=False)
                offsets[(r, h)] = [(int(p), np.sort(rng.choice(cfg.d, size=8, replace=False)).tolist())
                                   for p in np.sort(pages)]
    return Workload(cfg=cfg, budgets=budgets, contexts=contexts, n=n,
                    retained_pos=retained_pos, offsets=offsets)
