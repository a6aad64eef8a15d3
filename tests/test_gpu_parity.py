"""GPU parity of the whole decode path against the fp64 oracle, through the
C ABI, on the five workloads (the two largest on seeded samples of requests
and layers, with the caches built at full size and the split map the bench
uses) and on edge cases."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_harness import (OUT_MAX_ABS, SCORE_TOL, Stats, assert_output_bar, check_layer,
                         require_gpu, say)
from non_uniform_sparse_amd import kvs
from non_uniform_sparse_amd.pipeline import DecodeStep, default_microbatches
from non_uniform_sparse_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def _full(name, microbatches=1, **ov):
    """The workload at full size (or with overrides); microbatches=None takes
    the bench's own default for it."""
    require_gpu()
    wl = make_workload(name, **ov)
    if microbatches is None:
        microbatches = default_microbatches(wl)
    say(f"[case] {name} {ov} building caches")
    step = DecodeStep(wl, device="cuda", microbatches=microbatches)
    say(f"[case] {name}: W={step.W} T={step.T} S[0]={step.S[0].tolist()}")
    return wl, step


@pytest.mark.parametrize("name", ["tiny_ragged", "llama8b_ragged", "flexicache_topk"])
def test_workload_full(name):
    wl, step = _full(name)
    st = Stats()
    qs = step.queries()
    for l in range(wl.cfg.L):
        check_layer(step, l, qs[l], range(wl.cfg.b), st)
    assert_output_bar(st, name)


# Full-size caches; every layer of a seeded sample of requests, in chunks of
# layers so that each case stays well under two minutes.
_SAMPLED = [
    ("longctx_skew", [0, 3], range(0, 16)),
    ("longctx_skew", [0, 3], range(16, 32)),
    ("gemma3_mixed", [0, 1, 32, 63], range(0, 12)),
    ("gemma3_mixed", [0, 1, 32, 63], range(12, 24)),
    ("gemma3_mixed", [0, 1, 32, 63], range(24, 36)),
    ("gemma3_mixed", [0, 1, 32, 63], range(36, 48)),
]


@pytest.mark.parametrize("name,requests,layers", _SAMPLED,
                         ids=[f"{n}-L{r.start}-{r.stop - 1}" for n, _, r in _SAMPLED])
def test_workload_sampled(name, requests, layers):
    """Full-size caches and the step as the bench runs it (its request
    micro-batches, each on a stream of its own); the sampled requests of
    every layer of the chunk against the oracle.  The chunk starting at
    layer 0 also replays the step as a captured graph and checks every
    layer's output bit for bit against the eager step."""
    wl, step = _full(name, microbatches=None)
    assert len(step.parts) > 1
    st = Stats()
    qs = step.queries()
    step.run(qs)                       # every layer runs, as in the bench
    torch.cuda.synchronize()
    for l in layers:
        check_layer(step, l, qs[l], requests, st)
    assert_output_bar(st, f"{name} layers {layers.start}..{layers.stop - 1}")
    if layers.start != 0:
        return
    step.run(qs)
    torch.cuda.synchronize()
    ref = [b.out.clone() for b in step.bufs]
    g = step.capture(qs)
    for b in step.bufs:
        b.out.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for l, b in enumerate(step.bufs):
        assert torch.equal(b.out, ref[l]), f"micro-batched graph differs on layer {l}"


def _split_rows(step, l):
    c = step.cfg
    T = int(step.S[l].sum())
    uniform = kvs.kvs_plan_split(np.ones((1, c.Hkv)), step.head_slot[l:l + 1], c.Hp, 0.0, T)[0]
    return {"planned": step.S[l], "uniform": uniform, "one": np.ones(c.G, dtype=np.int32),
            "many": np.full(c.G, 997, dtype=np.int32)}


@pytest.mark.parametrize("name", ["tiny_ragged", "flexicache_topk"])
def test_split_invariance(name):
    """The combined output does not depend on the split map."""
    wl, step = _full(name, **({"b": 6} if name == "flexicache_topk" else {}))
    q = step.queries()[0]
    if wl.cfg.topk:
        step.select(0, q)
    outs = {}
    c = wl.cfg
    for key, row in _split_rows(step, 0).items():
        need = kvs.kvs_decode_workspace_bytes(c.b, c.Hq, c.Hkv, c.d, row)
        if need > step.workspace.numel():
            step.workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
        outs[key] = step.attend(0, q, S_row=row).clone()
    torch.cuda.synchronize()
    for key, o in outs.items():
        diff = (o - outs["planned"]).abs().max().item()
        say(f"split {key}: max diff vs planned {diff:.2e}")
        assert diff <= 1e-5


@pytest.mark.parametrize("name", ["tiny_ragged", "flexicache_topk", "gemma3_mixed"])
def test_phases_equal_one_call(name):
    """kvs_decode_splits then kvs_decode_combine on the same workspace give
    bit for bit what one kvs_decode_attn call gives (the same kernels); the
    split phase alone leaves out untouched."""
    wl, step = _full(name, **({"b": 6} if name == "flexicache_topk" else
                              {"b": 8, "L": 2} if name == "gemma3_mixed" else {}))
    c = wl.cfg
    qs = step.queries()
    for l in range(c.L):
        if c.topk:
            step.select(l, qs[l])
        buf = step.bufs[l]
        sel = buf.sel if c.topk else None
        cnt = buf.sel_count if c.topk else None
        one = step.attend(l, qs[l]).clone()
        out = torch.full_like(one, float("nan"))
        step.workspace.fill_(0xFF)            # NaN partials if a phase wrote nothing
        args = (step.caches[l], qs[l], sel, cnt, c.topk or 0, step.S[l], step.scale,
                step.workspace, out)
        kvs.kvs_decode_splits(*args)
        torch.cuda.synchronize()
        assert torch.isnan(out).all(), "the split phase wrote out"
        kvs.kvs_decode_combine(*args)
        torch.cuda.synchronize()
        assert torch.equal(out, one), f"{name} layer {l}: phases differ from one call"
    say(f"{name}: split + combine calls equal kvs_decode_attn on {c.L} layer(s)")


def test_full_topk_equals_dense():
    """With K at least every head's page count, top-K attention is dense
    attention over all retained tokens -- bit for bit, since the selected
    list is every page in ascending order."""
    require_gpu()
    wl = make_workload("llama8b_ragged", b=3, N=1000)
    step = DecodeStep(wl, device="cuda")
    c = wl.cfg
    q = step.queries()[0]
    dense = step.attend(0, q).clone()
    cache = step.caches[0]
    maxpg = step.layouts[0].page_table.shape[2]
    scores = torch.empty((c.b, c.Hkv, maxpg), dtype=torch.float32, device="cuda")
    K = maxpg + 5
    sel = torch.empty((c.b, c.Hkv, K), dtype=torch.int32, device="cuda")
    cnt = torch.empty((c.b, c.Hkv), dtype=torch.int32, device="cuda")
    kvs.kvs_score_pages(cache, q, scores)
    kvs.kvs_topk_pages(scores, cache.seq_len, c.P, K, sel, cnt)
    out = torch.empty_like(dense)
    kvs.kvs_decode_attn(cache, q, sel, cnt, K, step.S[0], step.scale, step.workspace, out)
    torch.cuda.synchronize()
    npg = (cache.seq_len + 15) // 16
    assert torch.equal(cnt, npg)
    assert torch.equal(out, dense)


@pytest.mark.parametrize("Hp,d,Hq,dtype,n_list", [
    (4, 128, 32, "f16", [1, 16, 17, 31, 32, 33, 200, 5]),
    (1, 128, 16, "bf16", [1, 2, 15, 16, 64, 65, 300, 7]),
    (8, 256, 16, "bf16", [3, 16, 48, 49, 100, 1, 129, 40]),
    (2, 256, 64, "f16", [16, 1, 77, 90, 33, 18, 250, 2]),
    (4, 128, 8, "bf16", [40, 1, 16, 300, 64, 65, 17, 2]),
])
@pytest.mark.parametrize("topk", [None, 3])
def test_edge_cases(Hp, d, Hq, dtype, n_list, topk):
    """Single-token heads, page-boundary lengths, partial pages, every GQA
    width the kernels build, group sizes 1..8, K above and below the page
    counts, and split maps with more splits than units (empty splits)."""
    require_gpu()
    wl = make_workload("llama8b_ragged", b=2, N=400, Hq=Hq, d=d, dtype=dtype, Hp=Hp, topk=topk)
    wl.n[0, 0, :] = n_list
    wl.n[1, 0, :] = n_list[::-1]
    say(f"[case] edge Hp={Hp} d={d} Hq={Hq} {dtype} topk={topk} n={n_list}")
    c = wl.cfg
    for T in (c.G, c.G + 3, 64):
        step = DecodeStep(wl, device="cuda", T=T)
        st = Stats()
        check_layer(step, 0, step.queries()[0], range(c.b), st)
        assert_output_bar(st, f"edge T={T}")


@pytest.mark.parametrize("whole_group", [False, True])
@pytest.mark.parametrize("topk", [None, 2])
def test_null_page_entries(topk, whole_group):
    """Null (-1) page-table entries: the min-max builder leaves their blocks
    untouched, scoring gives them -inf, and decode leaves their tokens out.
    Page 0 of every group stays valid, except that with whole_group every
    page of request 1's group 1 is null: its heads attend nothing and their
    query heads get zero rows."""
    require_gpu()
    wl = make_workload("llama8b_ragged", b=2, N=400, Hq=32, d=128, dtype="f16", Hp=4, topk=topk)
    wl.n[0, 0, :] = [40, 1, 16, 300, 64, 65, 17, 2]
    wl.n[1, 0, :] = [100, 33, 250, 49, 16, 80, 5, 129]
    say(f"[case] null pages topk={topk} whole_group={whole_group}")
    c = wl.cfg
    step = DecodeStep(wl, device="cuda")
    cache, lay = step.caches[0], step.layouts[0]
    nulls = {(0, 0): [1], (0, 1): [2, 5], (1, 0): [3], (1, 1): [1, 7]}
    if whole_group:
        nulls[(1, 1)] = list(range(lay.page_table.shape[2]))
    pt = lay.page_table.copy()
    for (r, i), ps in nulls.items():
        pt[r, i, [p for p in ps if p < pt.shape[2]]] = -1
    cache.page_table.copy_(torch.from_numpy(pt))
    cache.minmax.view(torch.int16).fill_(0x7E00)
    kvs.kvs_build_minmax(cache)
    q = step.queries()[0]
    if topk:
        step.select(0, q)
    out = step.attend(0, q).cpu().numpy().astype(np.float64)
    mm = cache.minmax.double().cpu().numpy()
    q64 = q.double().cpu().numpy()
    buf = step.bufs[0]
    hit = empty = 0
    for r in range(c.b):
        for h in range(c.Hkv):
            pos = int(step.head_slot[0, h])
            gi, j = pos // c.Hp, pos % c.Hp
            n = int(wl.n[r, 0, h])
            npg = -(-n // c.P)
            null = sorted(p for p in nulls.get((r, gi), []) if p < npg)
            hit += len(null)
            K64, V64 = wl.head_kv(r, 0, h, pos, device="cuda")
            K64, V64 = K64.double().cpu().numpy(), V64.double().cpu().numpy()
            lo, hi = O.page_minmax(K64, c.P)
            m0 = int(lay.meta_base[r, h])
            for p in range(npg):
                blk = mm[m0 + p]
                if p in null:
                    assert np.all(np.isnan(blk)), f"null page written r={r} h={h} p={p}"
                else:
                    assert np.array_equal(blk[:, 0], lo[p]) and np.array_equal(blk[:, 1], hi[p])
            qg = q64[r, h * c.Gq:(h + 1) * c.Gq]
            if topk:
                s = buf.scores[r, h, :npg].cpu().numpy()
                assert np.all(np.isneginf(s[null]))
                keep = [p for p in range(npg) if p not in null]
                want = O.page_scores(qg, lo[keep], hi[keep])
                A = np.max(np.abs(qg[:, None, :] * lo[keep][None]).sum(-1) +
                           np.abs(qg[:, None, :] * hi[keep][None]).sum(-1), axis=0)
                assert np.all(np.abs(s[keep] - want) <= SCORE_TOL * A)
                cnt = int(buf.sel_count[r, h])
                got = buf.sel[r, h, :cnt].cpu().numpy()
                assert np.array_equal(got, O.topk_pages(s, topk))
                pages = np.array([p for p in got if p not in null], dtype=np.int64)
            else:
                pages = np.array([p for p in range(npg) if p not in null], dtype=np.int64)
            ref = O.decode_head(qg, K64, V64, pages, c.P, step.scale)
            err = float(np.abs(out[r, h * c.Gq:(h + 1) * c.Gq] - ref).max())
            assert err <= OUT_MAX_ABS, f"r={r} h={h} err={err}"
            if len(pages) == 0:
                assert np.all(out[r, h * c.Gq:(h + 1) * c.Gq] == 0.0)
                empty += 1
    assert hit >= 4, "the case should null some pages of real heads"
    assert empty == (c.Hp if whole_group else 0)


def test_deterministic():
    wl, step = _full("flexicache_topk", b=4)
    q = step.queries()[0]
    a = step.run_layer(0, q).clone()
    sel_a = step.bufs[0].sel.clone()
    b = step.run_layer(0, q).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(sel_a, step.bufs[0].sel)


@pytest.mark.parametrize("name,mb", [("flexicache_topk", 1), ("longctx_skew", 1),
                                     ("flexicache_topk", 3), ("longctx_skew", 2)])
def test_graph_replay_matches_eager(name, mb):
    """A captured step (one stream, or request micro-batches on streams of
    their own) replays to the eager result, every replay, with eager work
    and synchronisation in between."""
    ov = {"b": 6} if name == "flexicache_topk" else {"L": 3}
    wl, step = _full(name, microbatches=mb, **ov)
    qs = step.queries()
    step.run(qs)
    torch.cuda.synchronize()
    ref = [b.out.clone() for b in step.bufs]
    ref_sel = [b.sel.clone() if b.sel is not None else None for b in step.bufs]
    g = step.capture(qs)
    for rep in range(3):
        for b in step.bufs:
            b.out.fill_(float("nan"))
            if b.sel is not None:
                b.sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, b in enumerate(step.bufs):
            assert torch.equal(b.out, ref[l]), f"replay {rep} layer {l}"
            if b.sel is not None:
                assert torch.equal(b.sel, ref_sel[l])
        step.run(qs)                 # eager work between replays
        torch.cuda.synchronize()

