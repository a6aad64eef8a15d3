"""Host logic: ragged layout round trip, C-ABI exports, argument
validation (checked before any HIP call, so no GPU is needed) and the host
planner / clustering against the oracle."""

import ctypes
import math
import re
import os

import numpy as np
import pytest
import torch

import oracle as O
from non_uniform_sparse_amd import kvs
from non_uniform_sparse_amd.layout import build_caches, unpack_head
from non_uniform_sparse_amd.pipeline import splits_per_request, topk_cap
from non_uniform_sparse_amd.workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(kvs.LIB_PATH):
        pytest.skip("libkvs.so not built")
    return kvs.lib()


def test_header_symbols_exported():
    L = _lib()
    header = open(os.path.join(ROOT, "include", "kvs.h")).read()
    declared = set(re.findall(r"\b(kvs_[a-z_]+)\s*\(", header))
    assert declared == set(kvs.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_last_error_starts_empty_and_reports():
    _lib()
    with pytest.raises(kvs.KvsError) as e:
        kvs.kvs_plan_split(np.ones((1, 8)), np.zeros((1, 8), dtype=np.int32), 4, 0.0, 4)
    assert e.value.code == kvs.KVS_EINVAL and "permutation" in str(e.value)


@pytest.mark.parametrize("name,overrides", [
    ("tiny_ragged", {}),
    ("llama8b_ragged", dict(b=2, N=700)),
    ("flexicache_topk", dict(b=2, N=320)),
    ("gemma3_mixed", dict(b=2, L=10, N=3000)),
])
def test_layout_round_trip(name, overrides):
    wl = make_workload(name, **overrides)
    c = wl.cfg
    hs = np.stack([O.cluster_heads(wl.budgets[l], c.Hp) if c.clustered else np.arange(c.Hkv)
                   for l in range(c.L)])
    caches, layouts = build_caches(wl, hs, device="cpu")
    for l in range(c.L):
        lay = layouts[l]
        for r in range(c.b):
            for i in range(c.G):
                members = [h for h in range(c.Hkv) if hs[l, h] // c.Hp == i]
                k = O.group_page_count([wl.n[r, l, h] for h in members], c.P)
                row = lay.page_table[r, i]
                assert (row[:k] >= 0).all() and (row[k:] == -1).all()
            for h in range(c.Hkv):
                K, V = unpack_head(caches[l].kv, lay, r, h, c.P)
                K0, V0 = wl.head_kv(r, l, h, int(hs[l, h]))
                assert torch.equal(K, K0) and torch.equal(V, V0)
    # physical ids are distinct within a pool
    for lam in range(c.nbanks):
        ls = [l for l in range(c.L) if layouts[l].pool == lam]
        for r in range(c.b):
            used = np.concatenate([layouts[ls[0]].page_table[r, i][layouts[ls[0]].page_table[r, i] >= 0]
                                   for i in range(c.G)])
            assert len(np.unique(used)) == len(used)


# ------------------------------------------------------------- planner -------

@pytest.mark.parametrize("seed", range(3))
def test_cluster_heads_matches_oracle(seed):
    _lib()
    rng = np.random.default_rng(seed)
    B = rng.uniform(0.02, 1.0, (6, 8))
    B[0, 3] = B[0, 5]                        # a tie
    B[1] = 0.5                               # all equal
    got = kvs.kvs_cluster_heads(B, 4)
    for l in range(6):
        assert got[l].tolist() == O.cluster_heads(B[l], 4).tolist()


def test_plan_split_matches_oracle_random():
    _lib()
    rng = np.random.default_rng(0)
    for _ in range(2000):
        Hp = int(rng.choice([1, 2, 4]))
        G = int(rng.integers(1, 5))
        Hkv = Hp * G
        L = int(rng.integers(1, 3))
        B = rng.uniform(1e-6, 1.0, (L, Hkv))
        if rng.random() < 0.3:
            B = np.round(B * 4) / 4 + 0.25      # many equal loads
            B = np.minimum(B, 1.0)
        hs = np.stack([rng.permutation(Hkv) for _ in range(L)])
        T = int(rng.integers(G, 70))
        cap = float(rng.choice([0.0, 0.1, 0.37]))
        got = kvs.kvs_plan_split(B, hs, Hp, cap, T)
        want = O.plan_split(B, hs, Hp, cap, T)
        assert got.tolist() == want.tolist()


# splits per request of each workload's step on MI355X (as the bench logs them)
RUNNING_T = {"tiny_ragged": 284, "llama8b_ragged": 128, "flexicache_topk": 51,
             "longctx_skew": 512, "gemma3_mixed": 32}


@pytest.mark.parametrize("name", ["tiny_ragged", "llama8b_ragged", "flexicache_topk",
                                  "longctx_skew", "gemma3_mixed"])
def test_plan_split_matches_oracle_on_workloads(name):
    _lib()
    wl = make_workload(name)
    c = wl.cfg
    hs = kvs.kvs_cluster_heads(wl.budgets, c.Hp) if c.clustered else \
        np.tile(np.arange(c.Hkv, dtype=np.int32), (c.L, 1))
    cap = topk_cap(wl)
    # the splits per request each workload runs with: T from the rule the
    # step uses, with W = 2048 concurrent decode workgroups (MI355X: 256
    # compute units x 8 resident one-wave workgroups for every kernel
    # variant these workloads build), then halved and doubled
    units = (np.minimum(c.topk, -(-wl.n // c.P)) if c.topk else -(-wl.n // c.P))
    T_run = splits_per_request(2048, c.b, c.G, float(units.sum(axis=2).mean()))
    assert T_run == RUNNING_T[name]
    for T in (c.G, 7, 64, 1024, T_run, max(c.G, T_run // 2), 2 * T_run):
        T = max(T, c.G)
        assert kvs.kvs_plan_split(wl.budgets, hs, c.Hp, cap, T).tolist() == \
            O.plan_split(wl.budgets, hs, c.Hp, cap, T).tolist()


# --------------------------------------------------------- validation --------

class _FakeCache:
    """A descriptor with fake (never dereferenced) device pointers."""

    def __init__(self, **kw):
        f = dict(kv=0x10000, minmax=0x20000, meta_base=0x28000, page_table=0x30000,
                 seq_len=0x40000, head_slot=0x50000, b=1, Hq=32, Hkv=8, Hp=4, d=128, P=16,
                 max_group_pages=4, num_pages=8, num_meta=8, dtype=kvs.KVS_F16)
        f.update(kw)
        self.s = kvs.PagedKV(**f)


@pytest.mark.parametrize("kw,code", [
    (dict(kv=0), kvs.KVS_EINVAL),
    (dict(kv=0x10008), kvs.KVS_EINVAL),       # misaligned
    (dict(Hq=30), kvs.KVS_EINVAL),
    (dict(Hp=3), kvs.KVS_EINVAL),
    (dict(d=64), kvs.KVS_EUNSUPPORTED),
    (dict(P=32), kvs.KVS_EUNSUPPORTED),
    (dict(dtype=7), kvs.KVS_EUNSUPPORTED),
    (dict(Hq=24), kvs.KVS_EUNSUPPORTED),      # query group of 3
    (dict(b=0), kvs.KVS_EINVAL),
    (dict(meta_base=0), kvs.KVS_EINVAL),
    (dict(num_meta=0), kvs.KVS_EINVAL),
    (dict(b=2048, Hkv=8, Hq=32), kvs.KVS_EUNSUPPORTED),   # b*Hkv above the LDS scan
])
def test_validation_before_launch(kw, code):
    L = _lib()
    s = _FakeCache(**kw).s
    assert L.kvs_build_minmax(ctypes.byref(s), None) == code
    assert kvs.last_error()
    assert L.kvs_score_pages(ctypes.byref(s), 0x60000, 0x70000, None) == code


@pytest.mark.parametrize("name", ["kvs_decode_attn", "kvs_decode_splits", "kvs_decode_combine"])
def test_decode_validation(name):
    """The decode and its two phases as separate calls make the same checks,
    all before any HIP call."""
    L = _lib()
    fn = getattr(L, name)
    s = _FakeCache().s
    S = np.array([2, 2], dtype=np.int32)
    need = kvs.kvs_decode_workspace_bytes(1, 32, 8, 128, S)
    assert need == 1 * 32 * 2 * 128 * 4 + 256 + 2 * 256
    args = lambda **k: [ctypes.byref(s), k.get("q", 0x60000), k.get("sel", None), k.get("cnt", None),
                        k.get("K", 0), k.get("S", S).ctypes.data, ctypes.c_float(k.get("scale", 0.088)),
                        k.get("ws", 0x100000), k.get("wsb", need), k.get("out", 0x80000), None]
    assert fn(*args(wsb=need - 1)) == kvs.KVS_ENOSPC
    assert name in kvs.last_error()
    assert fn(*args(S=np.array([2, 0], dtype=np.int32))) == kvs.KVS_EINVAL
    assert fn(*args(sel=0x90000, cnt=None, K=4)) == kvs.KVS_EINVAL
    assert fn(*args(sel=0x90000, cnt=0xA0000, K=0)) == kvs.KVS_EINVAL
    assert fn(*args(scale=-1.0)) == kvs.KVS_EINVAL
    assert fn(*args(ws=0x100010)) == kvs.KVS_EINVAL   # workspace alignment
    assert fn(*args(q=0)) == kvs.KVS_EINVAL


def test_decode_noalloc_validation():
    """The no-allocation decode makes the same checks as kvs_decode_attn and
    rejects a shape whose workspace exceeds its per-device scratch, all
    before any HIP call."""
    L = _lib()
    S = np.array([2, 2], dtype=np.int32)
    args = lambda s, **k: [ctypes.byref(s), k.get("q", 0x60000), k.get("sel", None),
                           k.get("cnt", None), k.get("K", 0), k.get("S", S).ctypes.data,
                           ctypes.c_float(k.get("scale", 0.088)), k.get("out", 0x80000), None]
    s = _FakeCache().s
    assert L.kvs_decode_attn_noalloc(*args(s, S=np.array([2, 0], dtype=np.int32))) == kvs.KVS_EINVAL
    assert L.kvs_decode_attn_noalloc(*args(s, sel=0x90000, cnt=None, K=4)) == kvs.KVS_EINVAL
    assert L.kvs_decode_attn_noalloc(*args(s, scale=-1.0)) == kvs.KVS_EINVAL
    assert L.kvs_decode_attn_noalloc(*args(s, q=0)) == kvs.KVS_EINVAL
    assert L.kvs_decode_attn_noalloc(*args(s, out=0x80008)) == kvs.KVS_EINVAL
    # 64 requests x 16 query heads x d = 256: 63 splits per group fit, 64 do not
    big = _FakeCache(b=64, Hq=16, Hkv=8, Hp=4, d=256).s
    fits = kvs.kvs_decode_workspace_bytes(64, 16, 8, 256, np.array([63, 1], dtype=np.int32))
    over = kvs.kvs_decode_workspace_bytes(64, 16, 8, 256, np.array([64, 1], dtype=np.int32))
    assert fits <= kvs.NOALLOC_SCRATCH_BYTES < over
    rc = L.kvs_decode_attn_noalloc(*args(big, S=np.array([64, 1], dtype=np.int32)))
    assert rc == kvs.KVS_ENOSPC and "scratch" in kvs.last_error()


def test_topk_validation():
    L = _lib()
    ok = [0x1000, 0x2000, 16, 1, 8, 640, 64, 0x3000, 0x4000, None]
    bad = {7: 0, 2: 32, 5: 9000}
    for idx, val in bad.items():
        a = list(ok)
        a[idx - 1 if idx == 7 else idx] = val
    a = list(ok); a[6] = 0
    assert L.kvs_topk_pages(*a) == kvs.KVS_EINVAL
    a = list(ok); a[6] = 2000
    assert L.kvs_topk_pages(*a) == kvs.KVS_EINVAL
    a = list(ok); a[2] = 32
    assert L.kvs_topk_pages(*a) == kvs.KVS_EUNSUPPORTED
    a = list(ok); a[5] = 9000
    assert L.kvs_topk_pages(*a) == kvs.KVS_EUNSUPPORTED
    a = list(ok); a[0] = None
    assert L.kvs_topk_pages(*a) == kvs.KVS_EINVAL


def test_plan_validation():
    _lib()
    hs = np.tile(np.arange(8, dtype=np.int32), (1, 1))
    with pytest.raises(kvs.KvsError):
        kvs.kvs_plan_split(np.ones((1, 8)), hs, 4, 0.0, 1)          # T < G
    with pytest.raises(kvs.KvsError):
        kvs.kvs_plan_split(np.zeros((1, 8)), hs, 4, 0.0, 4)         # budget 0
    with pytest.raises(kvs.KvsError):
        kvs.kvs_plan_split(np.ones((1, 8)), hs, 3, 0.0, 4)          # Hkv % Hp
    with pytest.raises(kvs.KvsError):
        kvs.kvs_cluster_heads(np.full((1, 8), 1.5), 4)



# ------------------------------------------------ append and head subsets --

def test_append_and_subset_validation():
    L = _lib()
    s = _FakeCache().s
    heads = np.ones(8, dtype=np.uint8)
    assert L.kvs_append_kv(ctypes.byref(s), None, 0x60000, None) == kvs.KVS_EINVAL
    assert L.kvs_append_kv(ctypes.byref(s), 0x60008, 0x70000, None) == kvs.KVS_EINVAL  # misaligned
    assert L.kvs_append_kv(None, 0x60000, 0x70000, None) == kvs.KVS_EINVAL
    assert L.kvs_score_pages_heads(ctypes.byref(s), 0x60000, None, 0x70000, None) == kvs.KVS_EINVAL
    s_big = _FakeCache(Hkv=256, Hq=256, Hp=8).s
    big = np.ones(256, dtype=np.uint8)
    assert L.kvs_score_pages_heads(ctypes.byref(s_big), 0x60000, big.ctypes.data, 0x70000,
                                   None) == kvs.KVS_EUNSUPPORTED
    assert L.kvs_topk_pages_heads(0x10000, 0x20000, 16, 1, 8, 4, 2, None, 0x30000, 0x40000,
                                  None) == kvs.KVS_EINVAL
    assert L.kvs_topk_pages_heads(0x10000, 0x20000, 16, 1, 8, 4, 0, heads.ctypes.data, 0x30000,
                                  0x40000, None) == kvs.KVS_EINVAL
    assert kvs.last_error()


def test_select_validation():
    """kvs_select_pages checks what kvs_score_pages and kvs_topk_pages check,
    before any launch (the scores buffer may be NULL)."""
    L = _lib()
    s = _FakeCache().s
    sel, cnt = 0x80000, 0x90000
    assert L.kvs_select_pages(ctypes.byref(s), None, None, 4, sel, cnt, None) == kvs.KVS_EINVAL
    assert L.kvs_select_pages(ctypes.byref(s), 0x60008, None, 4, sel, cnt, None) == kvs.KVS_EINVAL
    assert L.kvs_select_pages(ctypes.byref(s), 0x60000, None, 4, None, cnt, None) == kvs.KVS_EINVAL
    assert L.kvs_select_pages(ctypes.byref(s), 0x60000, None, 4, sel, None, None) == kvs.KVS_EINVAL
    for K in (0, 1025):
        assert L.kvs_select_pages(ctypes.byref(s), 0x60000, None, K, sel, cnt,
                                  None) == kvs.KVS_EINVAL
    long_heads = _FakeCache(max_group_pages=8193).s
    assert L.kvs_select_pages(ctypes.byref(long_heads), 0x60000, None, 4, sel, cnt,
                              None) == kvs.KVS_EUNSUPPORTED
    bad = _FakeCache(Hp=3).s
    assert L.kvs_select_pages(ctypes.byref(bad), 0x60000, None, 4, sel, cnt, None) == kvs.KVS_EINVAL
    assert L.kvs_select_pages(None, 0x60000, None, 4, sel, cnt, None) == kvs.KVS_EINVAL
    assert "kvs_select_pages" in kvs.last_error()


def test_fused_selection_policy():
    """One launch only for layers whose heads all hold pages and are of
    similar length; never without a top-K."""
    from non_uniform_sparse_amd.pipeline import fused_selection
    from non_uniform_sparse_amd.workloads import make_workload
    assert fused_selection(make_workload("flexicache_topk", b=4, N=2048)) == [True]
    assert not any(fused_selection(make_workload("gemma3_mixed", b=8, L=4)))
    wl = make_workload("flexicache_topk", b=4, N=2048)
    wl.n[1, 0, 3] = 0
    assert fused_selection(wl) == [False]
    assert not any(fused_selection(make_workload("llama8b_ragged", b=2)))


def test_rerank_schedule_matches_oracle():
    """kvs_rerank_heads (and the loop's heads_due, which calls it) against
    the oracle's rerank_due, and its argument checks."""
    from non_uniform_sparse_amd.steps import heads_due
    stable = np.array([True, False, True, True, False, True, True, True])
    for period in (1, 4, 16):
        for t in range(40):
            want = [O.rerank_due(t, bool(s), period) for s in stable]
            assert kvs.kvs_rerank_heads(stable, t, period).tolist() == want
            assert heads_due(t, stable, period).tolist() == want
    L = _lib()
    st = np.ones(8, dtype=np.uint8)
    due = np.zeros(8, dtype=np.uint8)
    for args in [(st.ctypes.data, 8, -1, 16), (st.ctypes.data, 8, 0, 0), (st.ctypes.data, 0, 0, 16),
                 (None, 8, 0, 16)]:
        assert L.kvs_rerank_heads(*args, due.ctypes.data) == kvs.KVS_EINVAL
    assert L.kvs_rerank_heads(st.ctypes.data, 8, 0, 16, None) == kvs.KVS_EINVAL


def test_prefill_quota_matches_oracle():
    """kvs_prefill_quota bit for bit against the oracle's chunk_quota (exact
    rationals) on budgets that are short binary fractions, decimal fractions
    with long expansions, values just below and above such points, the
    smallest normal doubles and 1; prompts ending inside, at and before a
    chunk; and the quotas telescoping to ceil(B N)."""
    g = np.random.default_rng(21)
    special = [1.0, 0.5, 0.25, 0.1, 1 / 3, 2 / 3, 0.999999, np.nextafter(0.5, 0), np.nextafter(0.5, 1),
               np.nextafter(1.0, 0), 2.0 ** -30, 2.0 ** -1000, 5e-324 * 2 ** 60, 0.3, 0.7]
    for trial in range(60):
        Hkv = int(g.integers(1, 9))
        B = np.array([special[int(g.integers(len(special)))] if g.random() < 0.5 else
                      float(g.uniform(1e-6, 1.0)) for _ in range(Hkv)])
        b = int(g.integers(1, 5))
        N = g.integers(1, 40000, size=b).astype(np.int64)
        if trial % 7 == 0:
            N[0] = 2 ** 40                     # the largest context
        chunk = int(g.choice([1, 7, 2048, 4096, 65536]))
        for start in [0, chunk, 3 * chunk, int(N.max()) - 1, int(N.max()) + 5]:
            start = min(max(0, start), 2 ** 40)
            q = kvs.kvs_prefill_quota(B, N, start, chunk)
            for r in range(b):
                a, e = min(int(N[r]), start), min(int(N[r]), start + chunk)
                for h in range(Hkv):
                    assert q[r, h] == O.chunk_quota(float(B[h]), a, e), (B[h], a, e)
    # telescoping over a whole prompt
    B = np.array([0.1, 1 / 3, 0.999999, 1.0])
    N = np.array([1, 2047, 2048, 2049, 100003], dtype=np.int64)
    tot = sum(kvs.kvs_prefill_quota(B, N, k * 2048, 2048) for k in range(-(-int(N.max()) // 2048)))
    for r in range(len(N)):
        for h in range(len(B)):
            assert tot[r, h] == O.retained_count(float(B[h]), int(N[r]))
    L = _lib()
    q = np.zeros((2, 2), dtype=np.int32)
    good = (np.array([0.5, 0.5]), np.array([10, 10], dtype=np.int64))
    call = lambda B_, N_, start=0, chunk=4: L.kvs_prefill_quota(B_.ctypes.data, N_.ctypes.data, len(N_),
                                                                len(B_), start, chunk, q.ctypes.data)
    assert call(*good) == kvs.KVS_OK
    assert call(np.array([0.0, 0.5]), good[1]) == kvs.KVS_EINVAL
    assert call(np.array([1.5, 0.5]), good[1]) == kvs.KVS_EINVAL
    assert call(np.array([np.nan, 0.5]), good[1]) == kvs.KVS_EINVAL
    assert call(good[0], np.array([0, 10], dtype=np.int64)) == kvs.KVS_EINVAL
    assert call(*good, start=-1) == kvs.KVS_EINVAL
    assert call(*good, chunk=0) == kvs.KVS_EINVAL


# ------------------------------------------------------------ host tier --

def test_tier_validation_before_any_hip_call():
    """Every descriptor check of the host-tier calls comes before the pinned
    pointer query (the only HIP call ahead of the launch)."""
    L = _lib()
    s = _FakeCache(Hp=1).s
    tier = lambda **k: kvs.HostTier(**{**dict(host_kv=0x900000, host_base=0x10000,
                                              slot_page=0x20000, slot_phys=0x30000, slots=64,
                                              num_host_pages=100), **k})
    prom = lambda s_, t, K=64: L.kvs_promote_pages(ctypes.byref(s_), ctypes.byref(t), 0x40000,
                                                   0x50000, K, None, None, None)
    assert prom(_FakeCache(Hp=4).s, tier()) == kvs.KVS_EUNSUPPORTED        # needs one head per table
    assert prom(s, tier(slots=0)) == kvs.KVS_EINVAL
    assert prom(s, tier(slots=2000)) == kvs.KVS_EINVAL
    assert prom(s, tier(num_host_pages=0)) == kvs.KVS_EINVAL
    assert prom(s, tier(host_kv=0x900008)) == kvs.KVS_EINVAL              # misaligned
    assert prom(s, tier(slot_phys=0)) == kvs.KVS_EINVAL
    assert prom(s, tier(), K=65) == kvs.KVS_EINVAL                         # K > slots
    assert prom(s, tier(), K=0) == kvs.KVS_EINVAL
    assert prom(_FakeCache(Hp=1, max_group_pages=9000).s, tier()) == kvs.KVS_EUNSUPPORTED
    assert L.kvs_promote_pages(ctypes.byref(s), None, 0x40000, 0x50000, 64, None, None,
                               None) == kvs.KVS_EINVAL
    assert L.kvs_promote_pages(ctypes.byref(s), ctypes.byref(tier()), None, 0x50000, 64, None,
                               None, None) == kvs.KVS_EINVAL
    assert L.kvs_offload_pages(ctypes.byref(_FakeCache(Hp=2).s), ctypes.byref(tier()),
                               None) == kvs.KVS_EUNSUPPORTED
    assert L.kvs_offload_pages(ctypes.byref(s), None, None) == kvs.KVS_EINVAL
    assert "tier" in kvs.last_error()
