"""fp64 reference for every step of the decode path (test infrastructure only).

All floating-point inputs are converted exactly to float64 by the caller
(fp16 and bf16 values are exactly representable).  Integer work is done with
Python integers or exact rationals.  Functions are written per head / per
group so that each can be checked by eye against its definition; none is
blocked, fused or reordered beyond what its definition states.

Notation (shared with the pages): P tokens per page, Hp KV heads per ragged
page group, G = Hkv / Hp groups per layer, Gq = Hq / Hkv query heads per KV
head, n retained tokens of a head, np = ceil(n / P) logical pages of a head.
"""

from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Sequence, Tuple

import numpy as np

__all__ = [
    "retained_count",
    "cluster_heads",
    "group_members",
    "group_page_count",
    "page_minmax",
    "page_scores",
    "topk_pages",
    "split_weight",
    "plan_split_layer",
    "plan_split",
    "split_bounds",
    "split_of_unit",
    "page_token_ids",
    "attention",
    "attention_lse",
    "lse_combine",
    "group_units",
    "decode_group_split",
    "decode_head",
    "rerank_due",
    "layer_scoring_needed",
    "decode_head_steps",
    "chunk_quota",
    "top_tokens",
    "prefill_head",
    "rerank_promotion",
    "decode_head_rerank",
]


# ---------------------------------------------------------------------------
# Retention and grouping -- Tangram review, 3.1 Budget Reservation and
# 3.2 Ragged Paging.
# ---------------------------------------------------------------------------

def retained_count(budget: float, context: int) -> int:
    """Tokens a head keeps: the ceiling of B * N (Tangram review, 3.1, the
    Top(ceil(B N), s) selection rule), with B in (0, 1].

    Evaluated on the exact binary value of ``budget`` with rationals, so no
    floating-point rounding can move the ceiling.
    """
    b = Fraction(budget)
    if not (0 < b <= 1):
        raise ValueError("budget must lie in (0, 1]")
    if context < 1:
        raise ValueError("context must be >= 1")
    return math.ceil(b * context)


def cluster_heads(budgets: Sequence[float], Hp: int) -> np.ndarray:
    """Budget-aware clustering (Tangram review, 3.2): heads of similar
    retention share a page group.

    Reading used (the pages give no formula): order the KV heads of one layer
    by budget, largest first, equal budgets by lower head index; the head at
    sorted position ``pos`` goes to group ``pos // Hp``, slot ``pos % Hp``.
    Returns ``head_slot[h] = pos``.
    """
    Hkv = len(budgets)
    if Hkv % Hp:
        raise ValueError("Hkv must be a multiple of Hp")
    order = sorted(range(Hkv), key=lambda h: (-float(budgets[h]), h))
    head_slot = np.empty(Hkv, dtype=np.int64)
    for pos, h in enumerate(order):
        head_slot[h] = pos
    return head_slot


def group_members(head_slot: Sequence[int], Hp: int) -> List[List[int]]:
    """Heads of each group in slot order: group i holds slots [i*Hp, (i+1)*Hp)."""
    Hkv = len(head_slot)
    by_slot = [None] * Hkv
    for h, s in enumerate(head_slot):
        by_slot[int(s)] = h
    if any(x is None for x in by_slot):
        raise ValueError("head_slot must be a permutation")
    return [by_slot[i * Hp:(i + 1) * Hp] for i in range(Hkv // Hp)]


def group_page_count(n_of_heads: Sequence[int], P: int) -> int:
    """Pages a group is allocated: enough for its longest head (Tangram
    review, 3.2: each group is sized by the largest budget inside it)."""
    return -(-max(int(n) for n in n_of_heads) // P)


# ---------------------------------------------------------------------------
# Page metadata and scoring -- FlexiCache summary, Core method (Quest-style
# min-max key bound) and Key observations, assumption 2 (MinMax cache).
# ---------------------------------------------------------------------------

def page_token_ids(p: int, n: int, P: int) -> range:
    """Valid token positions of logical page p of a head holding n tokens."""
    return range(p * P, min(n, (p + 1) * P))


def page_minmax(K: np.ndarray, P: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-page, per-channel minimum and maximum of the keys.

    ``K`` is the head's retained keys [n][d] in float64.  Page p covers
    tokens [p*P, min(n, (p+1)*P)); a partial last page uses its valid tokens
    only.  Returns (kmin, kmax), each [np][d].
    """
    K = np.asarray(K, dtype=np.float64)
    n, d = K.shape
    npg = -(-n // P)
    kmin = np.empty((npg, d))
    kmax = np.empty((npg, d))
    for p in range(npg):
        rows = K[p * P:min(n, (p + 1) * P)]
        kmin[p] = rows.min(axis=0)
        kmax[p] = rows.max(axis=0)
    return kmin, kmax


def page_scores(q_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Quest-style page score of one KV head (FlexiCache summary, Core method).

    For query row g and page p the bound is sum_d max(q[g,d]*kmin[p,d],
    q[g,d]*kmax[p,d]), an upper bound on q[g]·k for every key k of the page.
    The head's score is the largest bound over the query heads of its GQA
    group (reading: the per-KV-head score is max-reduced over the group).
    No 1/sqrt(d) scale: a positive scale does not change the ranking.
    Returns s[np] in float64.
    """
    q = np.asarray(q_group, dtype=np.float64)
    lo = np.asarray(kmin, dtype=np.float64)
    hi = np.asarray(kmax, dtype=np.float64)
    # bound[g, p] for every query row g and page p; then the max over g.
    bound = np.stack([np.maximum(q[g] * lo, q[g] * hi).sum(axis=1)
                      for g in range(q.shape[0])])
    return bound.max(axis=0)


def topk_pages(scores: Sequence[float], K: int) -> np.ndarray:
    """Per-KV-head top-K page selection (FlexiCache summary, Core method).

    Keeps the min(K, np) pages with the largest score; equal scores go to the
    lower page index.  The kept pages are returned in ascending page order.
    The comparison is done in whatever precision ``scores`` carries (pass
    float32-rounded scores to decide in the kernel's precision).
    """
    if K < 1:
        raise ValueError("K must be >= 1")
    s = [float(x) for x in scores]
    ranked = sorted(range(len(s)), key=lambda p: (-s[p], p))
    return np.array(sorted(ranked[:min(K, len(s))]), dtype=np.int64)


# ---------------------------------------------------------------------------
# Ahead-of-time split plan -- Tangram review, 3.3 AOT Load Balancing.
# ---------------------------------------------------------------------------

def split_weight(budget: float, cap: float = 0.0) -> int:
    """Integer weight of a head: round(min(B, cap) * 2^20), halves rounded up.

    ``cap <= 0`` means no cap.  The 2^-20 grid lets the planner compare
    group loads exactly in integers.  Evaluated with exact rationals.
    """
    b = Fraction(budget)
    if cap > 0:
        b = min(b, Fraction(cap))
    return math.floor(b * (1 << 20) + Fraction(1, 2))


def plan_split_layer(phi: Sequence[int], T: int) -> List[int]:
    """Split counts of one layer's groups (Tangram review, 3.3).

    The pages state only the goal: workgroups are handed out in proportion to
    each group's aggregated budget, so bigger groups get more and the load per
    workgroup is even.  Reading used: highest-averages (D'Hondt)
    apportionment -- every group starts with one split; each further split
    goes to the group with the largest load per split phi_i / S_i, compared
    exactly as phi_i * S_j vs phi_j * S_i, equal loads to the lower index.
    """
    G = len(phi)
    if T < G:
        raise ValueError("T must be >= number of groups")
    S = [1] * G
    for _ in range(T - G):
        best = 0
        for i in range(1, G):
            if phi[i] * S[best] > phi[best] * S[i]:
                best = i
        S[best] += 1
    return S


def plan_split(budgets: np.ndarray, head_slot: np.ndarray, Hp: int,
               cap: float, T: int) -> np.ndarray:
    """Static split map S[L][G] (Tangram review, 3.3: one row per layer, one
    column per head group).  Group load phi_i = sum of its heads' weights."""
    budgets = np.asarray(budgets)
    L, Hkv = budgets.shape
    G = Hkv // Hp
    S = np.zeros((L, G), dtype=np.int64)
    for l in range(L):
        phi = [0] * G
        for h in range(Hkv):
            phi[int(head_slot[l][h]) // Hp] += split_weight(budgets[l][h], cap)
        S[l] = plan_split_layer(phi, T)
    return S


# ---------------------------------------------------------------------------
# Attention, split and combine -- FlexiCache summary, Core method (sparse
# flash-decoding over the selected pages).
# ---------------------------------------------------------------------------

def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Plain softmax attention of one query row over m tokens:
    softmax(scale * K q) V, in float64."""
    o, _ = attention_lse(q, K, V, scale)
    return o


def attention_lse(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                  scale: float) -> Tuple[np.ndarray, float]:
    """Attention of one query row plus the log of its softmax denominator.

    z_t = scale * q·k_t, m = max z, l = sum exp(z - m), o = sum exp(z - m) v / l,
    lse = m + ln l.  With no tokens the result is (0, -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1] if V.ndim == 2 else q.shape[0]), -math.inf
    z = scale * (K @ q)
    m = float(z.max())
    w = np.exp(z - m)
    ell = float(w.sum())
    return (w @ V) / ell, m + math.log(ell)


def lse_combine(parts: Sequence[Tuple[np.ndarray, float]]) -> Tuple[np.ndarray, float]:
    """Merge partial results of disjoint token sets: with M = max lse_s,
    o = sum exp(lse_s - M) o_s / sum exp(lse_s - M), lse = M + ln(sum ...).
    Parts with lse = -inf (no tokens) carry no weight; when every part is
    empty the merge is empty too, (0, -inf), as attention over no token is
    (``attention_lse``)."""
    if not parts:
        raise ValueError("no part to merge")
    live = [(o, lse) for o, lse in parts if lse != -math.inf]
    if not live:
        return np.zeros_like(np.asarray(parts[0][0], dtype=np.float64)), -math.inf
    M = max(lse for _, lse in live)
    num = sum(math.exp(lse - M) * np.asarray(o, dtype=np.float64) for o, lse in live)
    den = sum(math.exp(lse - M) for _, lse in live)
    return num / den, M + math.log(den)


def split_bounds(U: int, S: int) -> List[Tuple[int, int]]:
    """Unit ranges of S splits over U units: split s covers
    [floor(s U / S), floor((s+1) U / S))."""
    return [((s * U) // S, ((s + 1) * U) // S) for s in range(S)]


def split_of_unit(u: int, U: int, S: int) -> int:
    """The split whose range (as in ``split_bounds``) contains unit u,
    found by scanning the ranges."""
    for s, (a, b) in enumerate(split_bounds(U, S)):
        if a <= u < b:
            return s
    raise ValueError("unit out of range")


def group_units(attended: Sequence[Sequence[int]]) -> List[Tuple[int, int]]:
    """Work units of one (request, group): head-major over the group's slots,
    then the slot's attended pages in list order -> [(slot, page), ...]."""
    return [(j, int(p)) for j, pages in enumerate(attended) for p in pages]


def decode_group_split(q_slots: Sequence[np.ndarray], K_slots: Sequence[np.ndarray],
                       V_slots: Sequence[np.ndarray], attended: Sequence[Sequence[int]],
                       P: int, S: int, scale: float) -> List[np.ndarray]:
    """Split-K decode of one (request, group) with S splits, then LSE combine.

    q_slots[j] is [Gq][d] (the query heads of the head in slot j), K_slots[j]
    and V_slots[j] are that head's retained tokens [n_j][d], attended[j] its
    attended logical pages.  Split s processes its contiguous range of the
    head-major unit list; for every head it touches it produces a partial
    (o, lse) over that head's valid tokens in the range; the partials of each
    query head are then merged with ``lse_combine``; a head with no valid
    token in its attended pages gets zero rows.  Returns [Gq][d] per slot.
    """
    units = group_units(attended)
    U = len(units)
    out = []
    for j in range(len(q_slots)):
        n_j = K_slots[j].shape[0]
        rows = []
        for g in range(q_slots[j].shape[0]):
            parts = []
            for a, b in split_bounds(U, S):
                toks = [t for (jj, p) in units[a:b] if jj == j
                        for t in page_token_ids(p, n_j, P)]
                if toks:
                    parts.append(attention_lse(q_slots[j][g], K_slots[j][toks],
                                               V_slots[j][toks], scale))
            rows.append(lse_combine(parts)[0] if parts else
                        np.zeros(np.asarray(V_slots[j]).shape[1]))
        out.append(np.stack(rows))
    return out


def decode_head(q_group: np.ndarray, K: np.ndarray, V: np.ndarray,
                pages: Sequence[int], P: int, scale: float) -> np.ndarray:
    """Attention of a KV head's query group over the valid tokens of its
    attended pages (the result split-K + combine reaches up to rounding);
    zero rows when there is none.  Returns [Gq][d]."""
    n = K.shape[0]
    toks = [t for p in pages for t in page_token_ids(int(p), n, P)]
    return np.stack([attention(q_group[g], K[toks], V[toks], scale)
                     for g in range(q_group.shape[0])])


# ---------------------------------------------------------------------------
# Decoding over steps -- FlexiCache summary, Method (head classes and the
# stability-aware rerank schedule) and Key observations, assumption 2 (the
# MinMax cache stays on the GPU, so a page can be scored at any step).
# ---------------------------------------------------------------------------

def rerank_due(t: int, stable: bool, period: int = 16) -> bool:
    """Whether a head re-selects its top-K pages at decode step t.

    Unstable heads re-select at every step; stable heads once every
    ``period`` steps and reuse their previous selection in between.
    Reading: steps are counted from the first decode step (t = 0), which
    always selects since no earlier selection exists, so a stable head
    re-selects at t = 0, period, 2*period, ...
    """
    if t < 0 or period < 1:
        raise ValueError("t >= 0 and period >= 1 required")
    return (not stable) or t % period == 0


def layer_scoring_needed(t: int, stable: Sequence[bool], period: int = 16) -> bool:
    """A layer is scored at step t only if some head of it re-selects; a
    layer of stable heads skips scoring between its rerank steps.  This
    never changes a result: scores of heads that do not re-select are not
    used."""
    return any(rerank_due(t, bool(s), period) for s in stable)


def decode_head_steps(q_steps: np.ndarray, K0: np.ndarray, V0: np.ndarray,
                      k_new: np.ndarray, v_new: np.ndarray, stable: bool, K: int,
                      P: int, scale: float, period: int = 16):
    """One KV head decoded over T steps with the rerank schedule.

    Step t first appends token t (k_new[t], v_new[t]) to the head's keys and
    values (the token being decoded is part of the cache it attends), then,
    if ``rerank_due(t, stable, period)``, re-selects the top-K pages from the
    min-max bounds of the pages as they now stand; otherwise it keeps the
    pages chosen at its last rerank (pages created since are not attended
    until the next rerank).  It then attends the current valid tokens of its
    selected pages.

    q_steps [T][Gq][d], K0/V0 [n0][d], k_new/v_new [T][d], all float64.
    Returns (outputs [T][Gq][d], selections: list of T page arrays).
    """
    Kc = np.asarray(K0, dtype=np.float64)
    Vc = np.asarray(V0, dtype=np.float64)
    sel = None
    outs, sels = [], []
    for t in range(q_steps.shape[0]):
        Kc = np.concatenate([Kc, np.asarray(k_new[t], dtype=np.float64)[None]])
        Vc = np.concatenate([Vc, np.asarray(v_new[t], dtype=np.float64)[None]])
        if rerank_due(t, stable, period):
            kmin, kmax = page_minmax(Kc, P)
            sel = topk_pages(page_scores(q_steps[t], kmin, kmax), K)
        outs.append(decode_head(q_steps[t], Kc, Vc, sel, P, scale))
        sels.append(np.array(sel, dtype=np.int64))
    return np.stack(outs), sels


# ---------------------------------------------------------------------------
# Budget Reservation in chunked prefill -- Tangram review, 3.1: as each
# prefill chunk's K/V is computed, every head keeps its top tokens by a score
# s, Top(ceil(B N), s) in all, so the compressed footprint is fixed when the
# request is scheduled and nothing is reclaimed later.
# ---------------------------------------------------------------------------

def chunk_quota(budget: float, start: int, end: int) -> int:
    """Tokens a head keeps from the chunk covering positions [start, end) of
    its prompt.  Reading: the cumulative kept count after position x is
    ceil(B x) (retained_count), so a chunk keeps ceil(B end) - ceil(B start);
    over all chunks of an N-token prompt this telescopes to ceil(B N), and it
    never exceeds the chunk's length since B <= 1."""
    if not 0 <= start <= end:
        raise ValueError("0 <= start <= end required")
    before = 0 if start == 0 else retained_count(budget, start)
    return (0 if end == 0 else retained_count(budget, end)) - before


def top_tokens(scores: Sequence[float], k: int) -> np.ndarray:
    """Positions of the k largest scores, equal scores to the lower position,
    returned in ascending position (the order in which they are kept)."""
    if k < 0:
        raise ValueError("k must be >= 0")
    s = [float(x) for x in scores]
    ranked = sorted(range(len(s)), key=lambda t: (-s[t], t))
    return np.array(sorted(ranked[:min(k, len(s))]), dtype=np.int64)


def prefill_head(K_chunks: Sequence[np.ndarray], V_chunks: Sequence[np.ndarray],
                 s_chunks: Sequence[np.ndarray], budget: float):
    """The keys and values one head holds after a chunked prefill: for each
    chunk in order, its top chunk_quota tokens by score, in position order,
    appended after those kept from earlier chunks.  Returns (K, V) [n][d]."""
    keptK, keptV, start = [], [], 0
    for Kc, Vc, sc in zip(K_chunks, V_chunks, s_chunks):
        end = start + len(sc)
        idx = top_tokens(sc, chunk_quota(budget, start, end))
        keptK.append(np.asarray(Kc, dtype=np.float64)[idx])
        keptV.append(np.asarray(Vc, dtype=np.float64)[idx])
        start = end
    d = np.asarray(K_chunks[0]).shape[1]
    K = np.concatenate(keptK) if keptK else np.zeros((0, d))
    V = np.concatenate(keptV) if keptV else np.zeros((0, d))
    return K, V


# ---------------------------------------------------------------------------
# Tiered placement of stable heads -- FlexiCache summary, Method: a stable
# head keeps only its top-K pages on the GPU, the rest in host memory, and a
# rerank brings over only the pages newly promoted into its selection;
# unstable heads stay entirely on the GPU.  The min-max bounds of every page
# stay on the GPU (Key observations, assumption 2), so scoring never reads
# host memory.
# ---------------------------------------------------------------------------

def rerank_promotion(resident: Sequence[int], selection: Sequence[int]):
    """Pages a rerank moves for one stable head: promoted = selected and not
    resident (copied host -> GPU), demoted = resident and not selected
    (their GPU slots are freed).  Afterwards the resident set is the
    selection.  Returns (promoted, demoted), each ascending."""
    res, sel = set(int(p) for p in resident), set(int(p) for p in selection)
    return (np.array(sorted(sel - res), dtype=np.int64),
            np.array(sorted(res - sel), dtype=np.int64))


def decode_head_rerank(q_steps: np.ndarray, K: np.ndarray, V: np.ndarray, stable: bool,
                       Ktop: int, P: int, scale: float, period: int = 16):
    """One KV head decoded over T steps of a fixed cache with the rerank
    schedule (no tokens appended): on a rerank step it re-selects its top-K
    pages from the pages' bounds, otherwise it keeps the previous selection;
    every step attends its selection.  Where the pages live (GPU or host)
    does not change the result.  Returns (outputs [T][Gq][d], selections)."""
    kmin, kmax = page_minmax(np.asarray(K, dtype=np.float64), P)
    sel, outs, sels = None, [], []
    for t in range(q_steps.shape[0]):
        if rerank_due(t, stable, period):
            sel = topk_pages(page_scores(q_steps[t], kmin, kmax), Ktop)
        outs.append(decode_head(q_steps[t], K, V, sel, P, scale))
        sels.append(np.array(sel, dtype=np.int64))
    return np.stack(outs), sels
