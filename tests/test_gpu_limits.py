"""Parity at the library's size limits and on empty heads, through the C ABI.

The top-K keeps a head's scores in LDS, which caps a head at 8192 pages
(131072 tokens) and K at 1024; both limits are taken here, with heavy
score ties and -inf (null) pages in the top-K case, and end to end on a
request whose heads reach the page limit (so one head spans thousands of
units and its query rows merge hundreds of split partials).  At the other
end, heads holding no token at all (a cache before its first prefill
chunk)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from gpu_harness import Stats, assert_output_bar, check_layer, require_gpu, say
from non_uniform_sparse_amd import kvs
from non_uniform_sparse_amd.pipeline import DecodeStep
from non_uniform_sparse_amd.workloads import make_workload

pytestmark = pytest.mark.gpu

P = 16
MAX_PAGES = 8192     # pages of one head the top-K takes
MAX_K = 1024


@pytest.mark.parametrize("K", [1, 1000, MAX_K])
def test_topk_at_page_limit(K):
    """Scores on a quarter grid (thousands of equal values per head) with 5%
    -inf entries; page counts at the limit, one below it, a single page,
    exactly K pages and one more.  Selection, count and -1 padding are exact
    against the oracle's rule (largest first, equal scores to the lower
    page, ascending output)."""
    require_gpu()
    say(f"[case] topk at the page limit K={K}")
    g = np.random.default_rng(11)
    b, Hkv = 2, 4
    s = (np.round(g.standard_normal((b, Hkv, MAX_PAGES)) * 4) / 4).astype(np.float32)
    s[g.random(s.shape) < 0.05] = -np.inf
    n = np.array([[MAX_PAGES * P, MAX_PAGES * P - 5, 1, K * P],
                  [(K + 1) * P, 17, (MAX_PAGES - 1) * P, 1000 * P + 3]], dtype=np.int32)
    dev = "cuda"
    scores = torch.from_numpy(s).to(dev)
    seq = torch.from_numpy(n).to(dev)
    sel = torch.full((b, Hkv, K), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((b, Hkv), -7, dtype=torch.int32, device=dev)
    kvs.kvs_topk_pages(scores, seq, P, K, sel, cnt)
    torch.cuda.synchronize()
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    for r in range(b):
        for h in range(Hkv):
            npg = -(-int(n[r, h]) // P)
            want = O.topk_pages(s[r, h, :npg], K)
            assert cnt_h[r, h] == len(want) == min(K, npg)
            assert np.array_equal(sel_h[r, h, :len(want)], want), f"r={r} h={h}"
            assert np.all(sel_h[r, h, len(want):] == -1)


@pytest.mark.parametrize("K", [1, 7, 64, MAX_K])
def test_topk_short_rows_with_ties(K):
    """Rows from empty to 1500 pages (around the 64- and 1024-item sizes),
    with scores from a three-value set (ties everywhere), an all-equal row, a
    row of -inf only and 5% -inf entries.  Exact against the oracle's rule."""
    require_gpu()
    say(f"[case] topk short rows K={K}")
    g = np.random.default_rng(12 + K)
    lens = [0, 1, 2, 63, 64, 65, 127, 640, 1000, 1023, 1024, 1025, 1500, 17, 5, 300]
    b, Hkv, maxpg = 2, 8, 1536
    s = g.choice(np.array([-1.5, 0.25, 3.0], dtype=np.float32), size=(b, Hkv, maxpg))
    s[g.random(s.shape) < 0.05] = -np.inf
    s[0, 3, :] = 0.5                       # all equal
    s[1, 6, :] = -np.inf                   # nothing but -inf
    n = np.array(lens, dtype=np.int32).reshape(b, Hkv) * P
    n[1, 0] -= 3                           # a partial last page
    dev = "cuda"
    scores = torch.from_numpy(s).to(dev)
    seq = torch.from_numpy(n).to(dev)
    sel = torch.full((b, Hkv, K), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((b, Hkv), -7, dtype=torch.int32, device=dev)
    kvs.kvs_topk_pages(scores, seq, P, K, sel, cnt)
    torch.cuda.synchronize()
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    for r in range(b):
        for h in range(Hkv):
            npg = -(-int(n[r, h]) // P)
            want = O.topk_pages(s[r, h, :npg], K)
            assert cnt_h[r, h] == len(want) == min(K, npg)
            assert np.array_equal(sel_h[r, h, :len(want)], want), f"r={r} h={h} npg={npg}"
            assert np.all(sel_h[r, h, len(want):] == -1)


@pytest.mark.parametrize("topk", [None, MAX_K])
def test_longest_heads_end_to_end(topk):
    """One request whose heads hold 1 to 131072 tokens (8192 pages): min-max
    build, scores, top-K with the largest K, split-K decode and combine, all
    against the oracle."""
    require_gpu()
    wl = make_workload("llama8b_ragged", b=1, N=MAX_PAGES * P, Hq=16, d=128, dtype="bf16",
                       Hp=2, topk=topk)
    wl.n[0, 0, :] = [MAX_PAGES * P, MAX_PAGES * P - 1, 1, 17, 65537, 100000, 2, MAX_PAGES * P - P]
    say(f"[case] longest heads topk={topk} n={wl.n[0, 0].tolist()}")
    step = DecodeStep(wl, device="cuda")
    assert step.layouts[0].page_table.shape[2] == MAX_PAGES
    st = Stats()
    check_layer(step, 0, step.queries()[0], [0], st)
    assert st.minmax_checked == sum(-(-int(x) // P) for x in wl.n[0, 0])
    assert_output_bar(st, f"longest heads topk={topk} S={step.S[0].tolist()}")


@pytest.mark.parametrize("topk", [None, 3])
def test_heads_without_tokens(topk):
    """Heads with n = 0, among them every head of one request's group and a
    whole request: no page, an all -inf score row, an empty selection
    (count 0, -1 padding), zero output rows; the other heads match the
    oracle as usual."""
    require_gpu()
    wl = make_workload("llama8b_ragged", b=3, N=400, Hq=32, d=128, dtype="f16", Hp=2, topk=topk)
    wl.n[0, 0, :] = [0, 40, 1, 0, 300, 17, 64, 0]
    wl.n[1, 0, :] = [0, 0, 0, 0, 0, 0, 0, 0]
    wl.n[2, 0, :] = [16, 0, 33, 250, 0, 5, 2, 129]
    say(f"[case] heads without tokens topk={topk}")
    step = DecodeStep(wl, device="cuda")
    c = wl.cfg
    st = Stats()
    check_layer(step, 0, step.queries()[0], range(c.b), st)
    assert_output_bar(st, f"heads without tokens topk={topk}")
    out = step.bufs[0].out.cpu().numpy()
    for r in range(c.b):
        for h in range(c.Hkv):
            if wl.n[r, 0, h] == 0:
                assert np.all(out[r, h * c.Gq:(h + 1) * c.Gq] == 0.0), f"r={r} h={h}"
    if topk:
        cnt = step.bufs[0].sel_count.cpu().numpy()
        assert np.array_equal(cnt == 0, wl.n[:, 0, :] == 0)


def test_long_runs_of_empty_heads():
    """Scoring deals all heads' pages out evenly, and a wave that finishes a
    head looks for the next one that holds pages, 64 heads per probe: here
    runs of 8, 63, 64, 65 and 130 heads without tokens (whole requests of 8
    heads, and a run cut inside a request) lie between heads that hold 1 to
    60 pages, so shares start, end and resume on both sides of every run.
    Scores, selections and outputs against the oracle."""
    require_gpu()
    b, Hkv = 48, 8
    wl = make_workload("llama8b_ragged", b=b, N=960, Hq=32, d=128, dtype="bf16", Hp=2, topk=5)
    g = np.random.default_rng(31)
    n = g.integers(1, 961, size=(b, Hkv))
    flat = n.reshape(-1)
    for lo, run in [(3, 8), (20, 63), (100, 64), (180, 65), (250, 130)]:
        flat[lo:lo + run] = 0
    flat[90] = 1          # a single-token head between two runs
    wl.n[:, 0, :] = flat.reshape(b, Hkv)
    say(f"[case] long runs of empty heads: {int((flat == 0).sum())} empty of {flat.size}")
    step = DecodeStep(wl, device="cuda")
    st = Stats()
    check_layer(step, 0, step.queries()[0], range(b), st)
    assert_output_bar(st, "long runs of empty heads")


@pytest.mark.parametrize("b", [300, 2047])
def test_scoring_at_many_heads(b):
    """b * Hkv = 2 400 and 16 376 heads (the documented limit is 16 383):
    the scoring kernel's page-count scan then loops over several batches of
    heads, and at the limit its LDS holds 64 KB of prefix.  Short heads
    (0 to 64 tokens), top-2; scores, selections and outputs of a seeded
    sample of requests against the oracle."""
    require_gpu()
    Hkv = 8
    wl = make_workload("llama8b_ragged", b=b, N=64, Hq=32, d=128, dtype="bf16", Hp=2, topk=2)
    g = np.random.default_rng(41)
    wl.n[:, 0, :] = g.integers(0, 65, size=(b, Hkv))
    say(f"[case] scoring at {b * Hkv} heads")
    step = DecodeStep(wl, device="cuda")
    st = Stats()
    sample = sorted(set([0, 1, b // 2, b - 2, b - 1] + g.integers(0, b, size=12).tolist()))
    check_layer(step, 0, step.queries()[0], sample, st)
    assert_output_bar(st, f"scoring at {b * Hkv} heads")

