"""GPU parity of tiered placement -- bulk offload, promotion after reranks,
decode over a cache whose stable heads keep only their selection on the GPU
-- against the fp64 oracle and the fully resident cache, through the C ABI.

Checked at every step, for every (request, layer, head):
  - offload: each tiered head's host pages hold its keys and values as the
    seeded generator drew them (bit-exact);
  - after promotion the head's resident set is exactly its selection, each
    resident page's table entry is its slot's physical page and its GPU copy
    is bit-equal to the host page; every other page is KVS_PAGE_ON_HOST;
  - the count of pages moved equals the oracle's promotion set difference;
  - selections and outputs equal those of the same schedule on the fully
    resident cache bit for bit, and outputs match the oracle's attention
    over the selected pages.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_harness import BAND, OUT_MAX_ABS, require_gpu, say
from non_uniform_sparse_amd.kvs import KVS_PAGE_ON_HOST
from non_uniform_sparse_amd.tiered import TieredLoop
from non_uniform_sparse_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def _stable(c):
    """Both kinds of head in every layer: heads 1 and Hkv-2 unstable."""
    s = np.ones((c.L, c.Hkv), dtype=bool)
    s[:, [1, c.Hkv - 2]] = False
    return s


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.view(torch.int16).cpu().numpy()


CASES = [
    ("flexicache_topk", dict(b=3, N=2000, Hp=1), 9, 4, None),
    ("flexicache_topk", dict(b=2, N=300, Hp=1), 5, 2, 70),        # fewer pages than K, spare slots
    ("gemma3_mixed", dict(b=3, L=2, N=4096, topk=16, Hp=1), 7, 3, None),
]


@pytest.mark.parametrize("name,ov,steps,period,slots", CASES)
def test_tier_steps_parity(name, ov, steps, period, slots):
    require_gpu()
    wl = make_workload(name, **ov)
    c = wl.cfg
    say(f"[case] tier {name} {ov} steps={steps} period={period} slots={slots}")
    stable = _stable(c)
    tl = TieredLoop(wl, steps, period=period, slots=slots, stable=stable)
    ref = TieredLoop(wl, steps, period=period, tiered=False, stable=stable)
    npg_all = -(-wl.n // c.P)                                         # [b][L][Hkv]
    for l in range(c.L):   # the compacted pool: unstable heads' pages plus the stable heads' slots
        want = int(npg_all[:, l, ~stable[l]].sum()) + c.b * int(stable[l].sum()) * tl.slots
        assert tl.tier_layouts[l].gpu_pages == want
    host = {}
    for l in range(c.L):
        lay, tier = tl.tier_layouts[l], tl.tiers[l]
        hk = _bits(tier.host_kv)
        for r in range(c.b):
            for h in range(c.Hkv):
                K, V = wl.head_kv(r, l, h, int(tl.ds.head_slot[l, h]), device="cuda")
                host[(l, r, h)] = (K.double().cpu().numpy(), V.double().cpu().numpy())
                hb = int(lay.host_base[r, h])
                assert (hb >= 0) == bool(stable[l, h])
                if hb < 0:
                    continue
                n = K.shape[0]
                npg = -(-n // c.P)
                pages = hk[hb:hb + npg]                               # [npg][2][P][d]
                kb, vb = _bits(K), _bits(V)
                for p in range(npg):
                    m = min(c.P, n - p * c.P)
                    assert np.array_equal(pages[p, 0, :m], kb[p * c.P:p * c.P + m]), (l, r, h, p)
                    assert np.array_equal(pages[p, 1, :m], vb[p * c.P:p * c.P + m]), (l, r, h, p)
    resident_prev = {k: np.zeros(0, dtype=np.int64) for k in host}
    total_moved, worst = 0, 0.0
    for t in range(steps):
        tl.run_step(t)
        ref.run_step(t)
        torch.cuda.synchronize()
        for l in range(c.L):
            buf, rbuf = tl.ds.bufs[l], ref.ds.bufs[l]
            assert torch.equal(buf.sel_count, rbuf.sel_count) and torch.equal(buf.sel, rbuf.sel), \
                f"selection differs from the resident cache t={t} l={l}"
            assert torch.equal(buf.out, rbuf.out), f"output differs from the resident cache t={t} l={l}"
            cache, tier, lay = tl.ds.caches[l], tl.tiers[l], tl.tier_layouts[l]
            pt = cache.page_table.cpu().numpy()
            kvb = _bits(cache.kv)
            hk = _bits(tier.host_kv)
            sp, sph = tier.slot_page.cpu().numpy(), tier.slot_phys.cpu().numpy()
            moved = tl.moved[l].cpu().numpy()
            sel, cnt = buf.sel.cpu().numpy(), buf.sel_count.cpu().numpy()
            scores = buf.scores.cpu().numpy()
            out = buf.out.cpu().numpy().astype(np.float64)
            q = tl.q[t][l].double().cpu().numpy()
            due = tl.heads_due(t, l)
            promoted = bool((due & stable[l]).any())   # else `moved` holds an earlier step's counts
            for r in range(c.b):
                for h in range(c.Hkv):
                    K, V = host[(l, r, h)]
                    npg = -(-K.shape[0] // c.P)
                    got = sel[r, h, :cnt[r, h]]
                    qg = q[r, h * c.Gq:(h + 1) * c.Gq]
                    if due[h]:   # the selection against the oracle's, up to near-ties
                        lo, hi = O.page_minmax(K, c.P)
                        s_ora = O.page_scores(qg, lo, hi)
                        assert np.array_equal(got, O.topk_pages(scores[r, h, :npg], c.topk))
                        fresh = O.topk_pages(s_ora.astype(np.float32), c.topk)
                        if not np.array_equal(got, fresh):
                            tau = float(np.sort(s_ora)[::-1][min(c.topk, npg) - 1])
                            for p in set(got.tolist()) ^ set(fresh.tolist()):
                                assert abs(s_ora[p] - tau) <= BAND * abs(tau), f"t={t} p={p}"
                    err = float(np.abs(out[r, h * c.Gq:(h + 1) * c.Gq] -
                                       O.decode_head(qg, K, V, got, c.P, tl.ds.scale)).max())
                    assert err <= OUT_MAX_ABS, f"t={t} l={l} r={r} h={h} err={err}"
                    worst = max(worst, err)
                    hb = int(lay.host_base[r, h])
                    if hb < 0:
                        assert not promoted or moved[r, h] == 0
                        continue
                    res = sp[r, h][sp[r, h] >= 0]
                    assert sorted(res.tolist()) == sorted(got.tolist()), f"resident set t={t} r={r} h={h}"
                    if promoted:
                        want = len(O.rerank_promotion(resident_prev[(l, r, h)], got)[0]) if due[h] else 0
                        assert moved[r, h] == want, f"moved t={t} l={l} r={r} h={h}"
                        total_moved += int(moved[r, h])
                    resident_prev[(l, r, h)] = res
                    row = pt[r, int(tl.ds.head_slot[l, h])]
                    for j in np.nonzero(sp[r, h] >= 0)[0]:
                        p, ph = int(sp[r, h, j]), int(sph[r, h, j])
                        assert row[p] == ph
                        assert np.array_equal(kvb[ph, 0], hk[hb + p]), f"slot copy t={t} p={p}"
                    others = np.setdiff1d(np.arange(npg), res)
                    assert np.all(row[others] == KVS_PAGE_ON_HOST)
    say(f"tier {name}: pages moved {total_moved}, GPU KV {tl.gpu_bytes / 2**20:.1f} MiB vs "
        f"{ref.full_bytes / 2**20:.1f} MiB resident, max-abs {worst:.2e}")
    assert total_moved > 0


def test_tier_unusable_slot_and_head_subset():
    """A slot whose physical id is out of range is never used; with one such
    slot and slots = K + 1 the selection still fits.  Heads outside the mask
    keep their state."""
    require_gpu()
    wl = make_workload("flexicache_topk", b=2, N=2000, Hp=1)
    c = wl.cfg
    say("[case] tier unusable slot")
    stable = np.ones((1, c.Hkv), dtype=bool)
    tl = TieredLoop(wl, 2, period=1, slots=c.topk + 1, stable=stable)
    tier = tl.tiers[0]
    tier.slot_phys[:, :, 0] = 1 << 30                 # outside the pool
    due = tl.select(0, 0)
    half = np.zeros(c.Hkv, dtype=bool)
    half[::2] = True
    buf = tl.ds.bufs[0]
    from non_uniform_sparse_amd import kvs
    kvs.kvs_promote_pages(tl.ds.caches[0], tier, buf.sel, buf.sel_count, c.topk, heads=half & due,
                          moved=tl.moved[0])
    torch.cuda.synchronize()
    sp = tier.slot_page.cpu().numpy()
    moved = tl.moved[0].cpu().numpy()
    cnt = buf.sel_count.cpu().numpy()
    assert np.all(sp[:, :, 0] == -1)
    for h in range(c.Hkv):
        if half[h]:
            assert np.all(moved[:, h] == cnt[:, h]) and np.all((sp[:, h] >= 0).sum(axis=1) == cnt[:, h])
        else:
            assert np.all(moved[:, h] == 0) and np.all(sp[:, h] == -1)


def test_tier_window_graph_matches_eager():
    """A captured window of steps (reranks with promotion, reuse, decode)
    replays to the eager result twice, each time from the rewound tier."""
    require_gpu()
    wl = make_workload("flexicache_topk", b=3, N=2000, Hp=1)
    say("[case] tier window graph")
    tl = TieredLoop(wl, 6, period=3, stable=_stable(wl.cfg))
    tl.rewind()
    for t in range(6):
        tl.run_step(t)
    torch.cuda.synchronize()
    ref_out = [o.clone() for o in tl.outputs()]
    ref_pt = [cc.page_table.clone() for cc in tl.ds.caches]
    ref_sp = [tr.slot_page.clone() for tr in tl.tiers]
    g = tl.capture(6)
    for rep in range(2):
        for o in tl.outputs():
            o.fill_(float("nan"))
        tl.rewind()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(wl.cfg.L):
            assert torch.equal(tl.outputs()[l], ref_out[l]), f"replay {rep} layer {l}"
            assert torch.equal(tl.ds.caches[l].page_table, ref_pt[l])
            assert torch.equal(tl.tiers[l].slot_page, ref_sp[l])


def test_tier_full_size_sampled():
    """flexicache_topk at full size (40 requests x 8 heads, 10240 tokens, top-64
    of 640 pages): one rerank window; outputs and selections equal the fully
    resident cache's, sampled heads match the oracle."""
    require_gpu()
    wl = make_workload("flexicache_topk", Hp=1)
    c = wl.cfg
    say("[case] tier full size")
    tl = TieredLoop(wl, 3, period=2)
    ref = TieredLoop(wl, 3, period=2, tiered=False, stable=tl.stable)
    rng = np.random.default_rng(5)
    for t in range(3):
        tl.run_step(t)
        ref.run_step(t)
        torch.cuda.synchronize()
        buf = tl.ds.bufs[0]
        assert torch.equal(buf.sel, ref.ds.bufs[0].sel) and torch.equal(buf.out, ref.ds.bufs[0].out)
        sel, cnt = buf.sel.cpu().numpy(), buf.sel_count.cpu().numpy()
        out = buf.out.cpu().numpy().astype(np.float64)
        q = tl.q[t][0].double().cpu().numpy()
        for _ in range(6):
            r, h = int(rng.integers(c.b)), int(rng.integers(c.Hkv))
            K, V = wl.head_kv(r, 0, h, int(tl.ds.head_slot[0, h]), device="cuda")
            K, V = K.double().cpu().numpy(), V.double().cpu().numpy()
            qg = q[r, h * c.Gq:(h + 1) * c.Gq]
            ora = O.decode_head(qg, K, V, sel[r, h, :cnt[r, h]], c.P, tl.ds.scale)
            assert np.abs(out[r, h * c.Gq:(h + 1) * c.Gq] - ora).max() <= OUT_MAX_ABS
    frac = tl.moved[0].sum().item()
    say(f"tier full size: GPU KV {tl.gpu_bytes / 2**30:.2f} GiB of {ref.full_bytes / 2**30:.2f} "
        f"GiB; pages moved on the last rerank {frac}")


@pytest.mark.parametrize("name,ov,steps,period", [
    ("flexicache_topk", dict(b=3, N=2000, Hp=1), 9, 4),
    ("gemma3_mixed", dict(b=3, L=2, N=4096, topk=16, Hp=1), 7, 3),
])
def test_tier_with_appends_matches_resident(name, ov, steps, period):
    """Decoding with appends on the tiered cache (rows written through to
    the host pages) against the same steps on the fully resident cache
    (DecodeLoop): lengths, bounds, selections and outputs equal bit for bit
    at every step; every tiered head's host pages hold all its tokens, old
    and appended; resident pages equal their host pages; the resident set is
    the selection."""
    from non_uniform_sparse_amd.steps import DecodeLoop
    require_gpu()
    wl = make_workload(name, **ov)
    c = wl.cfg
    say(f"[case] tier appends {name} {ov} steps={steps} period={period}")
    stable = _stable(c)
    tl = TieredLoop(wl, steps, period=period, stable=stable, append=True)
    ref = DecodeLoop(wl, steps, period=period, stable=stable)
    tokens = {}
    for l in range(c.L):
        for r in range(c.b):
            for h in range(c.Hkv):
                K, V = wl.head_kv(r, l, h, int(tl.ds.head_slot[l, h]), device="cuda")
                tokens[(l, r, h)] = [_bits(K), _bits(V)]
    for t in range(steps):
        tl.run_step(t)
        ref.run_step(t)
        torch.cuda.synchronize()
        for l in range(c.L):
            a, b_ = tl.ds, ref.ds
            assert torch.equal(a.caches[l].seq_len, b_.caches[l].seq_len)
            assert torch.equal(a.caches[l].minmax.view(torch.int16), b_.caches[l].minmax.view(torch.int16))
            assert torch.equal(a.bufs[l].sel, b_.bufs[l].sel) and torch.equal(a.bufs[l].sel_count,
                                                                              b_.bufs[l].sel_count)
            assert torch.equal(a.bufs[l].out, b_.bufs[l].out), f"output t={t} l={l}"
            tier, lay = tl.tiers[l], tl.tier_layouts[l]
            hk = _bits(tier.host_kv)
            kvb = _bits(a.caches[l].kv)
            pt = a.caches[l].page_table.cpu().numpy()
            sp, sph = tier.slot_page.cpu().numpy(), tier.slot_phys.cpu().numpy()
            sel, cnt = a.bufs[l].sel.cpu().numpy(), a.bufs[l].sel_count.cpu().numpy()
            kt, vt = [_bits(x) for x in tl.kv[t][l]]
            for r in range(c.b):
                for h in range(c.Hkv):
                    KV = tokens[(l, r, h)]
                    KV[0] = np.vstack([KV[0], kt[r, h][None]])
                    KV[1] = np.vstack([KV[1], vt[r, h][None]])
                    hb = int(lay.host_base[r, h])
                    if hb < 0:
                        continue
                    n = KV[0].shape[0]
                    for p in range(-(-n // c.P)):
                        m = min(c.P, n - p * c.P)
                        assert np.array_equal(hk[hb + p, 0, :m], KV[0][p * c.P:p * c.P + m]), (t, l, r, h, p)
                        assert np.array_equal(hk[hb + p, 1, :m], KV[1][p * c.P:p * c.P + m]), (t, l, r, h, p)
                    res = sp[r, h][sp[r, h] >= 0]
                    assert sorted(res.tolist()) == sorted(sel[r, h, :cnt[r, h]].tolist())
                    row = pt[r, int(tl.ds.head_slot[l, h])]
                    for j in np.nonzero(sp[r, h] >= 0)[0]:
                        p, ph = int(sp[r, h, j]), int(sph[r, h, j])
                        assert row[p] == ph and np.array_equal(kvb[ph, 0], hk[hb + p])
    say(f"tier appends {name}: {steps} steps equal to the resident cache")


def test_tier_appends_window_graph():
    """A captured window with appends and promotions replays, from the
    rewound state, to the eager result twice."""
    require_gpu()
    wl = make_workload("flexicache_topk", b=3, N=2000, Hp=1)
    say("[case] tier appends window graph")
    tl = TieredLoop(wl, 6, period=3, stable=_stable(wl.cfg), append=True)

    def state():
        return [(b.sel.clone(), b.out.clone(), cc.minmax.clone(), cc.seq_len.clone(),
                 cc.page_table.clone()) for b, cc in zip(tl.ds.bufs, tl.ds.caches)]

    tl.rewind()
    first = []
    for t in range(6):
        tl.run_step(t)
        torch.cuda.synchronize()
        first.append(state())
    tl.rewind()
    for t in range(6):       # a rewound window repeats the first at every step
        tl.run_step(t)
        torch.cuda.synchronize()
        for l, (want, got) in enumerate(zip(first[t], state())):
            for name, a, b in zip(("sel", "out", "minmax", "seq_len", "page_table"), want, got):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                    f"rewound step {t} layer {l}: {name} differs"   # bits: blocks past n hold NaN
    ref_out = [o.clone() for o in tl.outputs()]
    ref_len = [cc.seq_len.clone() for cc in tl.ds.caches]
    g = tl.capture(6)
    for rep in range(2):
        for o in tl.outputs():
            o.fill_(float("nan"))
        tl.rewind()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(wl.cfg.L):
            assert torch.equal(tl.outputs()[l], ref_out[l]), f"replay {rep} layer {l}"
            assert torch.equal(tl.ds.caches[l].seq_len, ref_len[l])
