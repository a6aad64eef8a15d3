"""GPU parity of decoding over steps -- append, stability-aware rerank and
selection reuse -- against the fp64 oracle, through the C ABI.

Every step of every (request, layer, head) is checked: the cache length
advanced by one, the page bounds equal the bounds of the grown keys
(value-exact), heads due for a rerank re-selected (exactly on the GPU's own
scores, and against the oracle's scores up to near-ties), the other heads
kept their previous selection unchanged, and the output equals the oracle's
attention over the current tokens of the selected pages."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_harness import BAND, OUT_MAX_ABS, require_gpu, say
from non_uniform_sparse_amd.steps import DecodeLoop
from non_uniform_sparse_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def _loop(name, ov, steps, period):
    require_gpu()
    wl = make_workload(name, **ov)
    loop = DecodeLoop(wl, steps, device="cuda", period=period)
    c = wl.cfg
    # force both kinds of layer: layer 0 all stable (skips scoring between
    # reranks), the others with two unstable heads
    loop.stable[:] = True
    for l in range(1, c.L):
        loop.stable[l, [1, c.Hkv - 2]] = False
    if c.L == 1:
        loop.stable[0, [1, c.Hkv - 2]] = False
    return wl, loop


@pytest.mark.parametrize("name,ov,steps,period", [
    ("flexicache_topk", dict(b=3, N=700), 10, 4),
    ("gemma3_mixed", dict(b=3, L=2, N=4096, topk=16), 9, 4),
])
def test_steps_parity(name, ov, steps, period):
    wl, loop = _loop(name, ov, steps, period)
    c = wl.cfg
    say(f"[case] steps {name} {ov} steps={steps} period={period}")
    host = {}
    for l in range(c.L):
        for r in range(c.b):
            for h in range(c.Hkv):
                K, V = wl.head_kv(r, l, h, int(loop.ds.head_slot[l, h]), device="cuda")
                host[(l, r, h)] = [K.double().cpu().numpy(), V.double().cpu().numpy()]
    prev = [None] * c.L
    worst, reused, reselected, stale = 0.0, 0, 0, 0
    for t in range(steps):
        loop.run_step(t)
        torch.cuda.synchronize()
        for l in range(c.L):
            kt, vt = [x.double().cpu().numpy() for x in loop.kv[t][l]]
            q = loop.q[t][l].double().cpu().numpy()
            cache, lay, buf = loop.ds.caches[l], loop.ds.layouts[l], loop.ds.bufs[l]
            seq = cache.seq_len.cpu().numpy()
            mm = cache.minmax.double().cpu().numpy()
            sel, cnt = buf.sel.cpu().numpy(), buf.sel_count.cpu().numpy()
            scores = buf.scores.cpu().numpy()
            out = buf.out.cpu().numpy().astype(np.float64)
            for r in range(c.b):
                for h in range(c.Hkv):
                    KV = host[(l, r, h)]
                    KV[0] = np.vstack([KV[0], kt[r, h][None]])
                    KV[1] = np.vstack([KV[1], vt[r, h][None]])
                    K, V = KV
                    n = K.shape[0]
                    assert seq[r, h] == n, f"t={t} l={l} r={r} h={h}"
                    lo, hi = O.page_minmax(K, c.P)
                    npg, m0 = lo.shape[0], int(lay.meta_base[r, h])
                    assert np.array_equal(mm[m0:m0 + npg, :, 0], lo), f"kmin t={t} l={l} r={r} h={h}"
                    assert np.array_equal(mm[m0:m0 + npg, :, 1], hi), f"kmax t={t} l={l} r={r} h={h}"
                    qg = q[r, h * c.Gq:(h + 1) * c.Gq]
                    got = sel[r, h, :cnt[r, h]]
                    s_ora = O.page_scores(qg, lo, hi)
                    fresh = O.topk_pages(s_ora.astype(np.float32), c.topk)
                    if O.rerank_due(t, bool(loop.stable[l, h]), period):
                        keep = min(c.topk, npg)
                        assert cnt[r, h] == keep
                        assert np.array_equal(got, O.topk_pages(scores[r, h, :npg], c.topk))
                        if not np.array_equal(got, fresh):
                            tau = float(np.sort(s_ora)[::-1][keep - 1])
                            for p in set(got.tolist()) ^ set(fresh.tolist()):
                                assert abs(s_ora[p] - tau) <= BAND * abs(tau), f"t={t} p={p}"
                        reselected += 1
                    else:
                        psel, pcnt = prev[l]
                        assert cnt[r, h] == pcnt[r, h] and np.array_equal(sel[r, h], psel[r, h]), \
                            f"selection changed without a rerank t={t} l={l} r={r} h={h}"
                        reused += 1
                        stale += int(not np.array_equal(got, fresh))
                    ref = O.decode_head(qg, K, V, got, c.P, loop.ds.scale)
                    err = float(np.abs(out[r, h * c.Gq:(h + 1) * c.Gq] - ref).max())
                    assert err <= OUT_MAX_ABS, f"t={t} l={l} r={r} h={h} err={err}"
                    worst = max(worst, err)
            prev[l] = (sel.copy(), cnt.copy())
    say(f"steps {name}: re-selections {reselected}, reuses {reused} "
        f"(stale vs a fresh rerank: {stale}), max-abs {worst:.2e}")
    assert reused > 0 and reselected > 0


def _step_state(loop):
    return [(b.sel.clone(), b.sel_count.clone(), b.scores.clone(), b.out.clone(),
             cc.minmax.clone(), cc.seq_len.clone()) for b, cc in zip(loop.ds.bufs, loop.ds.caches)]


def test_step_window_graph_matches_eager():
    """A rewound window repeats the first one exactly at every step (the
    selections, scores, outputs, bounds and lengths after each step; steps
    that score a page still filling would see the tokens of later steps if
    a rewind left the bounds behind), and a captured window replays to the
    eager result, twice in a row, each time from the rewound caches."""
    wl, loop = _loop("gemma3_mixed", dict(b=3, L=2, N=4096, topk=16), 6, 4)
    say("[case] step window graph")
    loop.rewind()
    first = []
    for t in range(6):
        loop.run_step(t)
        torch.cuda.synchronize()
        first.append(_step_state(loop))
    loop.rewind()
    for t in range(6):
        loop.run_step(t)
        torch.cuda.synchronize()
        for l, (want, got) in enumerate(zip(first[t], _step_state(loop))):
            for name, a, b in zip(("sel", "sel_count", "scores", "out", "minmax", "seq_len"),
                                  want, got):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                    f"rewound step {t} layer {l}: {name} differs"   # bits: blocks past n hold NaN
    ref = [o.clone() for o in loop.outputs()]
    ref_sel = [b.sel.clone() for b in loop.ds.bufs]
    ref_len = [cc.seq_len.clone() for cc in loop.ds.caches]
    g = loop.capture(6)
    for rep in range(2):
        for o in loop.outputs():
            o.fill_(float("nan"))
        loop.rewind()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(wl.cfg.L):
            assert torch.equal(loop.outputs()[l], ref[l]), f"replay {rep} layer {l}"
            assert torch.equal(loop.ds.bufs[l].sel, ref_sel[l])
            assert torch.equal(loop.ds.caches[l].seq_len, ref_len[l])
