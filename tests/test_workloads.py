"""The seeded generators draw what the workload recipes say."""

import numpy as np
import pytest
import torch

import oracle as O
from non_uniform_sparse_amd.workloads import CONFIGS, make_workload


@pytest.mark.parametrize("name", list(CONFIGS))
def test_retained_counts_match_oracle(name):
    wl = make_workload(name)
    c = wl.cfg
    for r in range(c.b):
        for l in range(c.L):
            for h in range(c.Hkv):
                assert wl.n[r, l, h] == O.retained_count(float(wl.budgets[l, h]), int(wl.contexts[r]))


def test_budget_recipes():
    assert np.all(make_workload("flexicache_topk").budgets == 1.0)
    wl = make_workload("longctx_skew")
    assert (wl.budgets == 1.0).sum() >= 26 and wl.budgets.min() >= 0.02
    wl = make_workload("gemma3_mixed")
    assert 2048 <= wl.contexts.min() and wl.contexts.max() <= 65536
    assert 0.4 < wl.budgets.mean() <= 0.5
    wl = make_workload("llama8b_ragged")
    assert wl.budgets.max() <= 1.0 and 0.45 < wl.budgets.mean() < 0.65


def test_tiny_retention_positions():
    wl = make_workload("tiny_ragged")
    for (r, l, h), pos in wl.retained_pos.items():
        assert len(pos) == wl.n[r, l, h] and np.all(np.diff(pos) > 0)
        assert pos[-1] < wl.cfg.N


def test_bank_prefix_views_are_deterministic():
    wl = make_workload("gemma3_mixed", b=2, L=16, N=4096)
    K1, V1 = wl.head_kv(1, 9, 3, pos=5)
    K2, V2 = wl.head_kv(1, 9, 3, pos=5)
    assert torch.equal(K1, K2) and torch.equal(V1, V2)
    # layers 1 and 9 share bank 1: the shorter view is a prefix of the longer
    Ka, _ = wl.head_kv(1, 1, 3, pos=5)
    m = min(Ka.shape[0], K1.shape[0])
    assert torch.equal(Ka[:m], K1[:m])


def test_offsets_shift_keys():
    wl = make_workload("flexicache_topk", b=1, N=640)
    K, _ = wl.head_kv(0, 0, 2, pos=2)
    page, chans = wl.offsets[(0, 2)][0]
    base = wl.bank(0, 0, 2)[:, 0]
    diff = (K[page * 16:(page + 1) * 16].float() - base[page * 16:(page + 1) * 16].float())
    assert torch.allclose(diff[:, chans], torch.full((16, 8), 3.0), atol=2e-2)
    other = [c for c in range(wl.cfg.d) if c not in chans]
    assert torch.all(diff[:, other] == 0)


def test_step_queries_drift_as_ar1():
    """Decode-step queries: q_0 is a fresh N(0,1) draw and every later q_t is
    rho q_{t-1} plus sqrt(1 - rho^2) of that step's fresh draw, so each q_t
    stays N(0,1) and consecutive queries correlate by rho; step_q(t) is the
    t-th element of the sequence."""
    from non_uniform_sparse_amd import workloads as W
    wl = make_workload("flexicache_topk", b=8, dtype="bf16")
    c = wl.cfg
    qs = wl.step_qs(12, 0)
    assert len(qs) == 12 and qs[0].shape == (c.b, c.Hq, c.d)
    assert torch.equal(wl.step_q(7, 0), qs[7])
    rho = W.QUERY_RHO
    # the recursion, in fp32 from the same fresh draws
    e = [torch.randn((c.b, c.Hq, c.d), generator=torch.Generator().manual_seed(
        W._mix(c.seed, 4, t, 0)), dtype=torch.float32) for t in range(12)]
    q = e[0]
    for t in range(1, 12):
        q = rho * q + (1 - rho * rho) ** 0.5 * e[t]
    assert torch.equal(qs[11], q.to(qs[11].dtype))
    # statistics over 8 x 32 x 128 values
    a, b = qs[10].float(), qs[11].float()
    assert abs(float(b.std()) - 1.0) < 0.02
    assert abs(float((a * b).mean()) / float((a * a).mean()) - rho) < 0.01
