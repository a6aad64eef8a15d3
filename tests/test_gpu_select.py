"""The one-launch score + top-K (kvs_select_pages) against the two calls it
replaces, through the C ABI: the same score bits, the same selections, the
same counts and -1 padding, for every head kind the library meets (null
page entries, heads without tokens, K above a head's page count, a head
with one page), both head sizes, both dtypes and every query-group size;
and end to end against the oracle on the FlexiCache-shaped workload, where
DecodeStep picks the fused launch by itself."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_harness import Stats, assert_output_bar, check_layer, require_gpu, say
from non_uniform_sparse_amd import kvs
from non_uniform_sparse_amd.pipeline import DecodeStep, fused_selection
from non_uniform_sparse_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def _both(step, K):
    """Separate calls and the fused one on layer 0; returns both results."""
    cache, q = step.caches[0], step.queries()[0]
    b, Hkv, maxpg = cache.page_table.shape[0], cache.seq_len.shape[1], cache.page_table.shape[2]
    dev = cache.kv.device
    out = []
    for fused in (False, True):
        scores = torch.full((b, Hkv, maxpg), 7.0, dtype=torch.float32, device=dev)
        sel = torch.full((b, Hkv, K), -7, dtype=torch.int32, device=dev)
        cnt = torch.full((b, Hkv), -7, dtype=torch.int32, device=dev)
        if fused:
            kvs.kvs_select_pages(cache, q, scores, K, sel, cnt)
        else:
            kvs.kvs_score_pages(cache, q, scores)
            kvs.kvs_topk_pages(scores, cache.seq_len, 16, K, sel, cnt)
        torch.cuda.synchronize()
        out.append((scores.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy()))
    # without a score buffer the selection is the same
    sel = torch.full((b, Hkv, K), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((b, Hkv), -7, dtype=torch.int32, device=dev)
    kvs.kvs_select_pages(cache, q, None, K, sel, cnt)
    torch.cuda.synchronize()
    out.append((None, sel.cpu().numpy(), cnt.cpu().numpy()))
    return out


def _assert_same(res, what):
    (s0, sel0, c0), (s1, sel1, c1), (_, sel2, c2) = res
    assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32)), f"{what}: scores differ"
    assert np.array_equal(sel0, sel1) and np.array_equal(c0, c1), f"{what}: selections differ"
    assert np.array_equal(sel0, sel2) and np.array_equal(c0, c2), f"{what}: selection w/o scores"


@pytest.mark.parametrize("d,dtype,Hq,Hkv,Hp", [
    (128, "f16", 32, 8, 2),     # Gq = 4
    (128, "bf16", 8, 8, 4),     # Gq = 1
    (256, "bf16", 16, 8, 2),    # Gq = 2
    (256, "f16", 64, 8, 8),     # Gq = 8
])
@pytest.mark.parametrize("K", [1, 5, 64])
def test_select_matches_score_then_topk(d, dtype, Hq, Hkv, Hp, K):
    require_gpu()
    say(f"[case] select d={d} {dtype} Hq={Hq} Hkv={Hkv} Hp={Hp} K={K}")
    wl = make_workload("llama8b_ragged", b=3, N=1500, Hq=Hq, d=d, dtype=dtype, Hp=Hp, topk=K)
    g = np.random.default_rng(5)
    wl.n[:, 0, :] = g.integers(1, 1500, size=(3, Hkv))
    wl.n[0, 0, :3] = [0, 1, 16]          # no token, one token, one full page
    wl.n[2, 0, -1] = 1500
    step = DecodeStep(wl, device="cuda")
    cache, lay = step.caches[0], step.layouts[0]
    pt = lay.page_table.copy()
    pt[1, 0, [0, 3, 4]] = -1              # null entries
    pt[2, pt.shape[1] - 1, 1::7] = -1
    cache.page_table.copy_(torch.from_numpy(pt))
    _assert_same(_both(step, K), f"d={d} {dtype} Gq={Hq // Hkv} K={K}")


def test_select_score_ties_and_long_heads():
    """Heads near the 8192-page limit whose bounds make many equal scores:
    the keys and the tie rule must agree with the two-launch path."""
    require_gpu()
    say("[case] select long heads with ties")
    wl = make_workload("llama8b_ragged", b=1, N=8192 * 16, Hq=16, d=128, dtype="bf16", Hp=2,
                       topk=1024)
    wl.n[0, 0, :] = [8192 * 16, 8191 * 16 + 3, 1, 17, 65537, 100000, 2, 1024 * 16]
    step = DecodeStep(wl, device="cuda")
    cache = step.caches[0]
    mm = cache.minmax
    mm.copy_((mm.float() * 4).round() / 4)   # a quarter grid: heavy ties
    _assert_same(_both(step, 1024), "long heads")


def test_fused_step_against_oracle():
    """flexicache_topk-shaped heads (all of one length): DecodeStep takes the
    fused launch, and selections and outputs meet the oracle's bar."""
    require_gpu()
    say("[case] fused step vs oracle")
    wl = make_workload("flexicache_topk", b=3, N=2048)
    assert all(fused_selection(wl))
    step = DecodeStep(wl, device="cuda")
    assert step.fused[0]
    st = Stats()
    check_layer(step, 0, step.queries()[0], range(wl.cfg.b), st)
    assert_output_bar(st, "fused flexicache step")


def test_select_rejects_bad_arguments():
    require_gpu()
    wl = make_workload("llama8b_ragged", b=1, N=64, Hq=8, d=128, dtype="f16", Hp=2, topk=4)
    step = DecodeStep(wl, device="cuda")
    cache, q = step.caches[0], step.queries()[0]
    Hkv = cache.seq_len.shape[1]
    for K in (0, 1025):
        sel = torch.zeros((1, Hkv, K), dtype=torch.int32, device="cuda")
        cnt = torch.zeros((1, Hkv), dtype=torch.int32, device="cuda")
        with pytest.raises(kvs.KvsError):
            kvs.kvs_select_pages(cache, q, None, K, sel, cnt)
