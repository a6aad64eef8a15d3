"""Pins of the fp64 oracle against things other than itself.

The pages print no worked numeric example, so the pins are: hand-worked
cases (tests/golden/hand_examples.json, each with its derivation), closed
forms, invariants that the pages state (the min-max score bounds q·k from
above; full-budget top-K is dense attention; the split-K combine does not
depend on the split count) and brute force on tiny inputs written in a
different form from the oracle's own code.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


# --------------------------------------------------------------- retention --

def _ceil_by_scan(b, N):
    """Smallest k >= 1 with k >= b*N, found by counting up (tiny N only)."""
    num, den = Fraction(b).numerator, Fraction(b).denominator
    k = 1
    while k * den < num * N:
        k += 1
    return k


@pytest.mark.parametrize("seed", range(5))
def test_retained_count_matches_scan(seed):
    rng = np.random.default_rng(seed)
    for _ in range(200):
        N = int(rng.integers(1, 300))
        b = float(rng.uniform(1e-3, 1.0))
        assert O.retained_count(b, N) == _ceil_by_scan(b, N)


def test_retained_count_closed_forms():
    assert O.retained_count(1.0, 4096) == 4096
    assert O.retained_count(0.5, 4096) == 2048
    assert O.retained_count(0.25, 17) == 5          # 4.25 -> 5
    assert O.retained_count(1e-9, 100) == 1         # never below one token
    # the stored double 0.1 is a hair above 1/10, so 10 * 0.1 is above 1
    assert Fraction(0.1) > Fraction(1, 10)
    assert O.retained_count(0.1, 10) == 2
    with pytest.raises(ValueError):
        O.retained_count(0.0, 10)
    with pytest.raises(ValueError):
        O.retained_count(1.5, 10)


# -------------------------------------------------------------- clustering --

def test_cluster_golden():
    g = GOLD["clustering"]
    hs = O.cluster_heads(g["budgets"], g["Hp"])
    assert hs.tolist() == g["head_slot"]
    groups = O.group_members(hs, g["Hp"])
    assert groups == [[1, 3, 6, 2], [7, 5, 0, 4]]
    assert math.isclose(sum(max(g["budgets"][h] for h in grp) for grp in groups),
                        g["sum_group_max"])


def _partitions(items, size):
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for combo in itertools.combinations(rest, size - 1):
        remaining = [x for x in rest if x not in combo]
        for tail in _partitions(remaining, size):
            yield [[first, *combo]] + tail


@pytest.mark.parametrize("Hkv,Hp", [(8, 4), (6, 2), (8, 2)])
def test_cluster_minimises_group_max_sum(Hkv, Hp):
    """Sorted grouping allocates the least memory (sum of group maxima) of
    every way of cutting the heads into groups of Hp -- brute force."""
    rng = np.random.default_rng(Hkv * 10 + Hp)
    for _ in range(20):
        B = rng.uniform(0.02, 1.0, Hkv)
        best = min(sum(max(B[h] for h in grp) for grp in part)
                   for part in _partitions(list(range(Hkv)), Hp))
        groups = O.group_members(O.cluster_heads(B, Hp), Hp)
        got = sum(max(B[h] for h in grp) for grp in groups)
        assert math.isclose(got, best, rel_tol=0, abs_tol=1e-15)


def test_group_page_count():
    assert O.group_page_count([16, 17, 1, 32], 16) == 2
    assert O.group_page_count([17], 16) == 2
    assert O.group_page_count([1, 1], 16) == 1
    assert O.group_page_count([4096, 100], 16) == 256


# ----------------------------------------------------------------- min-max --

@pytest.mark.parametrize("n", [1, 15, 16, 17, 40])
def test_minmax_bounds_are_tight(n):
    rng = np.random.default_rng(n)
    P, d = 16, 8
    K = rng.standard_normal((n, d))
    lo, hi = O.page_minmax(K, P)
    assert lo.shape == hi.shape == (-(-n // P), d)
    for p in range(lo.shape[0]):
        rows = K[p * P:min(n, (p + 1) * P)]
        for c in range(d):
            col = [float(x) for x in rows[:, c]]
            assert all(lo[p, c] <= x <= hi[p, c] for x in col)   # bound
            assert lo[p, c] in col and hi[p, c] in col           # attained


def test_minmax_single_token_page():
    K = np.array([[1.0, -2.0, 3.0]] * 16 + [[0.5, 0.25, -7.0]])
    lo, hi = O.page_minmax(K, 16)
    assert (lo[1] == K[16]).all() and (hi[1] == K[16]).all()


# ------------------------------------------------------------------- score --

def test_score_golden():
    g = GOLD["score_bound"]
    s = O.page_scores(np.array(g["q"]), np.array(g["kmin"]), np.array(g["kmax"]))
    assert s.tolist() == g["score"]
    q = np.array(g["q"])
    assert max(float(q[i] @ np.array(t)) for i in range(2) for t in g["tokens"]) == g["max_qk"]


def _score_by_corners(q, lo, hi):
    """max over query rows and over the 2^d corners of the key box of q·c."""
    best = -math.inf
    d = lo.shape[0]
    for g in range(q.shape[0]):
        for pick in itertools.product((0, 1), repeat=d):
            corner = np.where(np.array(pick) == 1, hi, lo)
            best = max(best, float(q[g] @ corner))
    return best


@pytest.mark.parametrize("Gq", [1, 2, 4])
def test_score_is_max_over_box_corners(Gq):
    rng = np.random.default_rng(Gq)
    d = 6
    for _ in range(30):
        q = rng.standard_normal((Gq, d))
        a, b = rng.standard_normal((2, 3, d))
        lo, hi = np.minimum(a, b), np.maximum(a, b)
        s = O.page_scores(q, lo, hi)
        for p in range(3):
            assert math.isclose(s[p], _score_by_corners(q, lo[p], hi[p]),
                                rel_tol=1e-12, abs_tol=1e-12)


def test_score_upper_bounds_every_token_and_is_tight_on_one_token():
    rng = np.random.default_rng(7)
    P, d, Gq = 16, 32, 4
    K = rng.standard_normal((16 * 5 + 1, d))
    q = rng.standard_normal((Gq, d))
    lo, hi = O.page_minmax(K, P)
    s = O.page_scores(q, lo, hi)
    for p in range(s.shape[0]):
        rows = K[p * P:min(K.shape[0], (p + 1) * P)]
        best = max(float(q[g] @ k) for g in range(Gq) for k in rows)
        A = max(float(np.abs(q[g] * lo[p]).sum() + np.abs(q[g] * hi[p]).sum()) for g in range(Gq))
        assert s[p] >= best - 1e-12 * A
    last = K[-1]
    assert math.isclose(s[-1], max(float(q[g] @ last) for g in range(Gq)), rel_tol=1e-12)


# -------------------------------------------------------------------- topk --

def test_topk_golden():
    for key in ("topk_ties", "topk_all"):
        g = GOLD[key]
        assert O.topk_pages(g["scores"], g["K"]).tolist() == g["selected"]


def _topk_by_rank(s, K):
    """Page p is kept iff fewer than K pages beat it, where q beats p when
    s_q > s_p, or s_q == s_p and q < p."""
    keep = []
    for p in range(len(s)):
        beaten_by = sum(1 for q in range(len(s)) if s[q] > s[p] or (s[q] == s[p] and q < p))
        if beaten_by < K:
            keep.append(p)
    return keep


@pytest.mark.parametrize("seed", range(4))
def test_topk_matches_rank_definition(seed):
    rng = np.random.default_rng(seed)
    for _ in range(100):
        npg = int(rng.integers(1, 40))
        K = int(rng.integers(1, 45))
        s = rng.integers(-3, 4, npg).astype(float)         # many ties
        if rng.random() < 0.3:
            s = rng.standard_normal(npg)
        assert O.topk_pages(s, K).tolist() == _topk_by_rank(s, K)


def test_topk_permutation_equivariant():
    rng = np.random.default_rng(11)
    s = rng.standard_normal(50)
    perm = rng.permutation(50)
    a = set(O.topk_pages(s, 7).tolist())
    b = set(perm[O.topk_pages(s[perm], 7)].tolist())
    assert a == b


# -------------------------------------------------------------------- plan --

def test_split_weight_closed_forms():
    assert O.split_weight(1.0) == 1 << 20
    assert O.split_weight(0.5) == 1 << 19
    assert O.split_weight(2.0 ** -21) == 1          # exactly half rounds up
    assert O.split_weight(2.0 ** -22) == 0          # a quarter rounds down
    assert O.split_weight(0.9, cap=0.25) == 1 << 18
    assert O.split_weight(0.1, cap=0.25) == round(0.1 * 2 ** 20)


def test_plan_golden():
    for key in ("plan_31", "plan_111"):
        g = GOLD[key]
        assert O.plan_split_layer(g["phi"], g["T"]) == g["S"]


def _compositions(T, G):
    for cut in itertools.combinations(range(1, T), G - 1):
        edges = (0, *cut, T)
        yield [edges[i + 1] - edges[i] for i in range(G)]


@pytest.mark.parametrize("G", [1, 2, 3, 4])
def test_plan_is_optimal_by_brute_force(G):
    """The plan minimises the largest load per split, max_i phi_i / S_i,
    over every way of giving each group at least one of the T splits."""
    rng = np.random.default_rng(G)
    for _ in range(40):
        phi = [int(x) for x in rng.integers(0, 1 << 20, G)]
        T = int(rng.integers(G, 17))
        S = O.plan_split_layer(phi, T)
        assert sum(S) == T and min(S) >= 1
        got = max(Fraction(phi[i], S[i]) for i in range(G))
        best = min(max(Fraction(phi[i], c[i]) for i in range(G)) for c in _compositions(T, G))
        assert got == best


def test_plan_monotone_in_T():
    phi = [5, 3, 2, 1]
    prev = O.plan_split_layer(phi, 4)
    for T in range(5, 40):
        cur = O.plan_split_layer(phi, T)
        assert all(c >= p for c, p in zip(cur, prev)) and sum(cur) == T
        prev = cur


def test_plan_split_uses_groups():
    B = np.array([[1.0, 0.25, 0.25, 0.5], [0.5, 0.5, 0.5, 0.5]])
    hs = np.array([[0, 1, 2, 3], [3, 2, 1, 0]])
    S = O.plan_split(B, hs, 2, 0.0, 6)
    # layer 0: groups {0,1}=1.25, {2,3}=0.75 -> loads 5:3 -> (4,2) (max 5/16 vs 3/8 for (3,3))
    # layer 1: equal loads -> (3,3)
    assert S.tolist() == [[4, 2], [3, 3]]


# --------------------------------------------------------- attention/combine --

def test_two_token_golden():
    g = GOLD["two_token_softmax"]
    o, lse = O.attention_lse(np.array(g["q"]), np.array(g["K"]), np.array(g["V"]), g["scale"])
    assert math.isclose(o[0], g["o"][0], rel_tol=1e-14)
    assert math.isclose(lse, g["lse"], rel_tol=1e-14)


def test_combine_golden():
    g = GOLD["combine_two"]
    o, lse = O.lse_combine([(np.array(p[0]), p[1]) for p in g["parts"]])
    assert np.allclose(o, g["o"], rtol=1e-14, atol=0)
    assert math.isclose(lse, g["lse"], rel_tol=1e-14)
    o2, _ = O.lse_combine([(np.array([9.0, 9.0]), -math.inf)] +
                          [(np.array(p[0]), p[1]) for p in g["parts"]])
    assert np.allclose(o2, g["o"], rtol=1e-14, atol=0)


def test_attention_closed_forms():
    rng = np.random.default_rng(3)
    d = 5
    k = rng.standard_normal((1, d))
    v = rng.standard_normal((1, d))
    q = rng.standard_normal(d)
    o, lse = O.attention_lse(q, k, v, 0.7)
    assert np.array_equal(o, v[0]) and math.isclose(lse, 0.7 * float(q @ k[0]))
    K = rng.standard_normal((9, d))
    V = rng.standard_normal((9, d))
    o, lse = O.attention_lse(np.zeros(d), K, V, 1.0)
    assert np.allclose(o, V.mean(axis=0), rtol=1e-13, atol=1e-15)
    assert math.isclose(lse, math.log(9))


def _attention_naive(q, K, V, scale):
    w = [math.exp(scale * sum(q[i] * K[t][i] for i in range(len(q)))) for t in range(len(K))]
    tot = sum(w)
    return [sum(w[t] * V[t][c] for t in range(len(K))) / tot for c in range(len(V[0]))]


def test_attention_brute_force_and_hull():
    rng = np.random.default_rng(5)
    for _ in range(50):
        d = int(rng.integers(1, 5))
        m = int(rng.integers(1, 7))
        q, K, V = rng.standard_normal(d), rng.standard_normal((m, d)), rng.standard_normal((m, d))
        o = O.attention(q, K, V, 1.0 / math.sqrt(d))
        assert np.allclose(o, _attention_naive(q, K, V, 1.0 / math.sqrt(d)), rtol=1e-12, atol=1e-14)
        assert (o >= V.min(axis=0) - 1e-14).all() and (o <= V.max(axis=0) + 1e-14).all()


def _group_case(rng, n_list, d=8, Gq=2):
    q = [rng.standard_normal((Gq, d)) for _ in n_list]
    K = [rng.standard_normal((n, d)) for n in n_list]
    V = [rng.standard_normal((n, d)) for n in n_list]
    return q, K, V


def test_split_invariance():
    """The combined result does not depend on the number of splits."""
    rng = np.random.default_rng(9)
    P = 4
    n_list = [23, 5, 13, 1]
    q, K, V = _group_case(rng, n_list)
    attended = [list(range(-(-n // P))) for n in n_list]
    U = sum(len(a) for a in attended)
    ref = O.decode_group_split(q, K, V, attended, P, 1, 0.35)
    for S in (2, 3, 7, U, U + 3):
        got = O.decode_group_split(q, K, V, attended, P, S, 0.35)
        for a, b in zip(ref, got):
            assert np.allclose(a, b, rtol=1e-12, atol=1e-14)
    direct = [O.decode_head(q[j], K[j], V[j], attended[j], P, 0.35) for j in range(4)]
    for a, b in zip(ref, direct):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_heads_without_tokens_give_zero_rows():
    """A head holding no token, and a head whose attended list is empty,
    attend nothing: zero rows (the empty softmax sum carries no weight), at
    every split count, while the group's other heads keep their dense
    result.  An all-empty merge is (0, -inf), like attention over no token."""
    rng = np.random.default_rng(21)
    P = 4
    n_list = [0, 9, 6, 3]
    q, K, V = _group_case(rng, n_list)
    attended = [[], [0, 1, 2], [], [0]]
    U = sum(len(a) for a in attended)
    for S in (1, 2, U, U + 2):
        got = O.decode_group_split(q, K, V, attended, P, S, 0.5)
        assert np.array_equal(got[0], np.zeros((2, 8)))
        assert np.array_equal(got[2], np.zeros((2, 8)))
        for j in (1, 3):   # every token of these heads is attended
            dense = np.array([_attention_naive(q[j][g], K[j], V[j], 0.5) for g in range(2)])
            assert np.allclose(got[j], dense, rtol=1e-12, atol=1e-14)
    assert np.array_equal(O.decode_head(q[0], K[0], V[0], [], P, 0.5), np.zeros((2, 8)))
    o, lse = O.lse_combine([(np.ones(3), -math.inf), (np.full(3, 5.0), -math.inf)])
    assert np.array_equal(o, np.zeros(3)) and lse == -math.inf
    with pytest.raises(ValueError):
        O.lse_combine([])


def test_full_budget_topk_is_dense():
    """With K >= np, attention over the selected pages is dense attention
    over every retained token."""
    rng = np.random.default_rng(21)
    P, d, Gq = 16, 16, 4
    K = rng.standard_normal((16 * 7 + 3, d))
    V = rng.standard_normal(K.shape)
    q = rng.standard_normal((Gq, d))
    lo, hi = O.page_minmax(K, P)
    sel = O.topk_pages(O.page_scores(q, lo, hi), 64)
    assert sel.tolist() == list(range(8))
    got = O.decode_head(q, K, V, sel, P, 0.25)
    for g in range(Gq):
        z = 0.25 * (K @ q[g])
        w = np.exp(z - z.max())
        assert np.allclose(got[g], (w / w.sum()) @ V, rtol=1e-12, atol=1e-15)


def test_topk_attention_sees_only_selected_pages():
    rng = np.random.default_rng(4)
    P, d = 4, 4
    K = rng.standard_normal((20, d))
    V = rng.standard_normal((20, d))
    q = rng.standard_normal((1, d))
    pages = [3, 1]
    got = O.decode_head(q, K, V, pages, P, 1.0)
    toks = [12, 13, 14, 15, 4, 5, 6, 7]
    assert np.allclose(got[0], _attention_naive(q[0], K[toks], V[toks], 1.0), rtol=1e-12)


def test_split_bounds_cover_units():
    for U in range(0, 30):
        for S in range(1, 12):
            b = O.split_bounds(U, S)
            assert b[0][0] == 0 and b[-1][1] == U
            assert all(b[i][1] == b[i + 1][0] for i in range(S - 1))
            sizes = [y - x for x, y in b]
            assert max(sizes) - min(sizes) <= 1
            for u in range(U):
                s = O.split_of_unit(u, U, S)
                assert b[s][0] <= u < b[s][1]


def test_split_bounds_floor_convention():
    # split s starts at floor(s U / S): 5 units over 3 splits -> sizes 1, 2, 2
    assert O.split_bounds(5, 3) == [(0, 1), (1, 3), (3, 5)]
    assert O.split_bounds(2, 4) == [(0, 0), (0, 1), (1, 1), (1, 2)]


# ------------------------------------------------ decoding over steps ------

def test_rerank_schedule_counts():
    """Stable heads re-select at t = 0, period, 2 period, ...; unstable heads
    every step; a layer of stable heads is scored only at those steps."""
    T = 48
    assert [t for t in range(T) if O.rerank_due(t, True, 16)] == [0, 16, 32]
    assert all(O.rerank_due(t, False, 16) for t in range(T))
    assert all(O.rerank_due(t, True, 1) for t in range(T))
    assert [t for t in range(T) if O.layer_scoring_needed(t, [True] * 8, 16)] == [0, 16, 32]
    assert all(O.layer_scoring_needed(t, [True] * 7 + [False], 16) for t in range(T))
    with pytest.raises(ValueError):
        O.rerank_due(-1, True)


@pytest.mark.parametrize("kind", ["stable", "unstable"])
def test_decode_steps_golden(kind):
    g = GOLD["rerank_reuse"]
    outs, sels = O.decode_head_steps(np.array(g["q_steps"]), np.array(g["K0"]), np.array(g["V0"]),
                                     np.array(g["k_new"]), np.array(g["v_new"]), kind == "stable",
                                     g["K"], g["P"], g["scale"], g["period"])
    assert np.allclose(outs[:, 0, 0], [o[0] for o in g[kind]["o"]], rtol=1e-14, atol=0)
    assert [s.tolist() for s in sels] == g[kind]["sel"]


def _dense(q, K, V, scale):
    z = (K @ q) * scale
    w = np.exp(z - z.max())
    return (w[:, None] * V).sum(axis=0) / w.sum()


def test_decode_steps_full_budget_every_step_is_dense():
    """With K covering every page and a re-selection at every step, each step
    is dense attention over all tokens held so far, the new one included."""
    rng = np.random.default_rng(5)
    P, d, Gq, T, n0 = 4, 3, 2, 9, 6
    K0, V0 = rng.normal(size=(n0, d)), rng.normal(size=(n0, d))
    kn, vn = rng.normal(size=(T, d)), rng.normal(size=(T, d))
    q = rng.normal(size=(T, Gq, d))
    outs, sels = O.decode_head_steps(q, K0, V0, kn, vn, False, 100, P, 0.7, 16)
    for t in range(T):
        Kt, Vt = np.vstack([K0, kn[:t + 1]]), np.vstack([V0, vn[:t + 1]])
        assert sels[t].tolist() == list(range(-(-(n0 + t + 1) // P)))
        for g in range(Gq):
            assert np.allclose(outs[t, g], _dense(q[t, g], Kt, Vt, 0.7), rtol=1e-12, atol=1e-14)


def test_decode_steps_stable_head_keeps_stale_pages():
    """Between reranks a stable head attends exactly the pages chosen at its
    last rerank, with the tokens those pages hold now; pages created later
    are not attended."""
    rng = np.random.default_rng(9)
    P, d, T, n0, K = 4, 2, 12, 7, 2
    K0, V0 = rng.normal(size=(n0, d)), rng.normal(size=(n0, d))
    kn, vn = rng.normal(size=(T, d)) + 4.0, rng.normal(size=(T, d))
    q = np.ones((T, 1, d))
    outs, sels = O.decode_head_steps(q, K0, V0, kn, vn, True, K, P, 1.0, 16)
    first = sels[0].tolist()
    assert all(s.tolist() == first for s in sels)
    for t in range(1, T):
        n = n0 + t + 1
        Kt, Vt = np.vstack([K0, kn[:t + 1]]), np.vstack([V0, vn[:t + 1]])
        toks = [i for p in first for i in range(p * P, min(n, (p + 1) * P))]
        assert np.allclose(outs[t, 0], _dense(q[t, 0], Kt[toks], Vt[toks], 1.0), rtol=1e-12)
    # an unstable head sees the new high-key pages instead
    _, sels_u = O.decode_head_steps(q, K0, V0, kn, vn, False, K, P, 1.0, 16)
    assert sels_u[-1].tolist() != first


# ------------------------------------------------ budget reservation -------

def test_chunk_budget_golden():
    g = GOLD["chunk_budget"]
    C, N, B = g["chunk"], g["N"], g["budget"]
    starts = list(range(0, N, C))
    assert [O.chunk_quota(B, a, min(N, a + C)) for a in starts] == g["quotas"]
    d = 1
    Ks = [np.arange(a, min(N, a + C), dtype=float)[:, None] for a in starts]   # K = global position
    Vs = [-k for k in Ks]
    K, V = O.prefill_head(Ks, Vs, [np.array(s) for s in g["scores"]], B)
    assert K[:, 0].tolist() == g["kept_global"] and V[:, 0].tolist() == [-x for x in g["kept_global"]]


@pytest.mark.parametrize("B,N,C", [(0.3, 1000, 64), (1.0, 77, 16), (0.01, 5000, 512),
                                   (0.577, 32768, 2048), (1 / 3, 99, 7)])
def test_chunk_quotas_telescope_to_the_budget(B, N, C):
    """Summed over the chunks, the quotas are ceil(B N), each at most the
    chunk's length (the footprint is fixed when the request is scheduled)."""
    q = [O.chunk_quota(B, a, min(N, a + C)) for a in range(0, N, C)]
    assert sum(q) == O.retained_count(B, N)
    assert all(0 <= x <= min(C, N - a) for x, a in zip(q, range(0, N, C)))


def test_prefill_one_chunk_full_budget_and_brute_force():
    """B = 1 keeps every token; on tiny chunks the selection equals the brute
    force over all subsets of the quota's size (maximal score sum, then the
    lexicographically smallest positions among equal sums)."""
    import itertools
    rng = np.random.default_rng(2)
    K = rng.normal(size=(12, 3)); V = rng.normal(size=(12, 3))
    s = rng.integers(0, 4, size=12).astype(float)          # many ties
    Kf, Vf = O.prefill_head([K], [V], [s], 1.0)
    assert np.array_equal(Kf, K) and np.array_equal(Vf, V)
    for k in range(0, 6):
        best = max(itertools.combinations(range(12), k),
                   key=lambda c: (sum(s[list(c)]), [-t for t in c]))
        assert O.top_tokens(s, k).tolist() == list(best)


# ------------------------------------------------ tiered placement ---------

def test_rerank_promotion_sets():
    """After a rerank the resident set is the selection: promoted and the
    kept pages make up the selection, demoted and kept the old residents."""
    rng = np.random.default_rng(4)
    for _ in range(200):
        npg = int(rng.integers(1, 60))
        old = rng.choice(npg, size=int(rng.integers(0, npg + 1)), replace=False)
        new = rng.choice(npg, size=int(rng.integers(0, npg + 1)), replace=False)
        pro, dem = O.rerank_promotion(old, new)
        kept = set(old.tolist()) & set(new.tolist())
        assert set(pro.tolist()) | kept == set(new.tolist()) and not set(pro.tolist()) & kept
        assert set(dem.tolist()) | kept == set(old.tolist()) and not set(dem.tolist()) & kept
        assert list(pro) == sorted(pro) and list(dem) == sorted(dem)
    assert O.rerank_promotion([], [3, 1])[0].tolist() == [1, 3]          # first rerank
    assert O.rerank_promotion([2, 5], [2, 5])[0].size == 0                 # nothing moves


def test_decode_rerank_stable_head_keeps_pages_between_reranks():
    """Hand-checkable: two single-token pages, K = 1.  The query points at
    page 0 on step 0 and at page 1 on step 1; a stable head (period 2) keeps
    page 0 on step 1, an unstable one moves; on step 2 both re-select."""
    K = np.array([[1.0], [-1.0]]); V = np.array([[10.0], [20.0]])
    q = np.array([[[1.0]], [[-1.0]], [[-1.0]]])
    o_s, s_s = O.decode_head_rerank(q, K, V, True, 1, 1, 1.0, period=2)
    o_u, s_u = O.decode_head_rerank(q, K, V, False, 1, 1, 1.0, period=2)
    assert [s.tolist() for s in s_s] == [[0], [0], [1]]
    assert [s.tolist() for s in s_u] == [[0], [1], [1]]
    assert o_s[:, 0, 0].tolist() == [10.0, 10.0, 20.0] and o_u[:, 0, 0].tolist() == [10.0, 20.0, 20.0]
