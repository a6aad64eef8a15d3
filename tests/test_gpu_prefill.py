"""GPU parity of the chunked prefill under Budget Reservation against the
fp64 oracle, through the C ABI: after every chunk of every layer, each head
holds exactly the oracle's kept tokens (bit for bit, in order, in its ragged
pages), its length is ceil(B N) at the end, its page bounds are value-exact,
and a decode step on the prefilled cache matches the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_harness import BAND, OUT_MAX_ABS, require_gpu, say
from non_uniform_sparse_amd.layout import unpack_head
from non_uniform_sparse_amd.prefill import ChunkedPrefill
from non_uniform_sparse_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,ov,C", [
    ("llama8b_ragged", dict(b=2, N=1000), 256),
    ("gemma3_mixed", dict(b=3, L=2, N=4096, topk=16), 512),
    ("llama8b_ragged", dict(b=2, N=700, Hp=2, dtype="bf16"), 100),
    ("longctx_skew", dict(b=1, L=2, N=600), 8),        # small budgets: chunks that keep nothing
    ("llama8b_ragged", dict(b=1, N=20000), 8192),      # the longest chunk the call takes
])
def test_prefill_parity(name, ov, C):
    require_gpu()
    wl = make_workload(name, **ov)
    c = wl.cfg
    say(f"[case] prefill {name} {ov} C={C}")
    pf = ChunkedPrefill(wl, C, device="cuda")
    host = {}
    for k in range(pf.chunks):
        for l in range(c.L):
            kc, vc, s = pf.inputs(l, k)
            host[(l, k)] = (kc.double().cpu().numpy(), vc.double().cpu().numpy(),
                            s.double().cpu().numpy())
            pf.run_chunk(l, k, inputs=(kc, vc, s))
    torch.cuda.synchronize()
    zero_quota = 0
    for l in range(c.L):
        cache, lay = pf.ds.caches[l], pf.ds.layouts[l]
        seq = cache.seq_len.cpu().numpy()
        mm = cache.minmax.double().cpu().numpy()
        for r in range(c.b):
            N = int(wl.contexts[r])
            for h in range(c.Hkv):
                Ks, Vs, Ss = [], [], []
                for k in range(pf.chunks):
                    valid = min(C, N - k * C)
                    if valid <= 0:
                        break
                    kc, vc, s = host[(l, k)]
                    Ks.append(kc[r, h, :valid]), Vs.append(vc[r, h, :valid]), Ss.append(s[r, h, :valid])
                    zero_quota += int(O.chunk_quota(float(wl.budgets[l, h]), k * C, k * C + valid) == 0)
                Kref, Vref = O.prefill_head(Ks, Vs, Ss, float(wl.budgets[l, h]))
                n = Kref.shape[0]
                assert n == O.retained_count(float(wl.budgets[l, h]), N) == seq[r, h]
                Kg, Vg = unpack_head(cache.kv, lay, r, h, c.P)
                assert np.array_equal(Kg.double().cpu().numpy(), Kref), f"K l={l} r={r} h={h}"
                assert np.array_equal(Vg.double().cpu().numpy(), Vref), f"V l={l} r={r} h={h}"
                lo, hi = O.page_minmax(Kref, c.P)
                m0 = int(lay.meta_base[r, h])
                assert np.array_equal(mm[m0:m0 + lo.shape[0], :, 0], lo)
                assert np.array_equal(mm[m0:m0 + lo.shape[0], :, 1], hi)
                host[("kv", l, r, h)] = (Kref, Vref)
    # a decode step on the prefilled cache
    worst = 0.0
    for l in range(c.L):
        q = pf.ds.queries()[l]
        out = pf.ds.run_layer(l, q).cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
        q64 = q.double().cpu().numpy()
        buf = pf.ds.bufs[l]
        for r in range(c.b):
            for h in range(c.Hkv):
                Kref, Vref = host[("kv", l, r, h)]
                qg = q64[r, h * c.Gq:(h + 1) * c.Gq]
                if c.topk:
                    cnt = int(buf.sel_count[r, h])
                    pages = buf.sel[r, h, :cnt].cpu().numpy()
                    lo, hi = O.page_minmax(Kref, c.P)
                    s_ora = O.page_scores(qg, lo, hi)
                    ref_sel = O.topk_pages(s_ora.astype(np.float32), c.topk)
                    if not np.array_equal(pages, ref_sel):
                        tau = float(np.sort(s_ora)[::-1][cnt - 1])
                        for p in set(pages.tolist()) ^ set(ref_sel.tolist()):
                            assert abs(s_ora[p] - tau) <= BAND * abs(tau)
                else:
                    pages = np.arange(-(-Kref.shape[0] // c.P))
                ref = O.decode_head(qg, Kref, Vref, pages, c.P, pf.ds.scale)
                err = float(np.abs(out[r, h * c.Gq:(h + 1) * c.Gq] - ref).max())
                assert err <= OUT_MAX_ABS, f"decode l={l} r={r} h={h} err={err}"
                worst = max(worst, err)
    say(f"prefill {name}: chunks {pf.chunks}, zero-quota chunks {zero_quota}, decode max-abs {worst:.2e}")
    if C == 8:
        assert zero_quota > 0
