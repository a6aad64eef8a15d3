"""Decode-attention benchmark on one MI355X.

A step is one full decode step of the workload: for every layer, page
scores -> top-K pages (top-K workloads only) -> ragged split-K decode + LSE
combine, captured once as a HIP graph and replayed (the requests may be cut
into micro-batches whose layer chains run on streams of their own).  Inputs
(caches, min-max metadata, queries) are resident in HBM before the timed
region starts.  The roofline object is the dominant kernel's, the split-K
decode timed alone in whole-batch launches; every other kernel of the path
has a row of its own.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from non_uniform_sparse_amd import kvs  # noqa: E402
from non_uniform_sparse_amd.pipeline import DecodeStep, default_microbatches  # noqa: E402
from non_uniform_sparse_amd.workloads import CONFIGS, make_workload  # noqa: E402

METRIC = "decode-attn KV GB/s (% of HBM peak) + µs/step, ragged top-K, 1 MI355X"
HBM_PEAK_GBPS = 8000.0
DEFAULT_CONFIG = "gemma3_mixed"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(step: DecodeStep, l: int) -> dict:
    """Bytes the method itself must move in layer l (not the dense work it
    avoids).  KV: 2*d*s per valid token of every attended page.  Metadata:
    2*d*s per valid page (top-K only).  Small terms: q, scores, selection,
    split partials (written + read) and the output."""
    c, wl = step.cfg, step.wl
    s = 2
    n = wl.n[:, l, :]                                       # [b][Hkv]
    npg = -(-n // c.P)
    if c.topk:
        sel = step.bufs[l].sel.cpu().numpy()
        cnt = step.bufs[l].sel_count.cpu().numpy()
        toks = 0
        for r in range(c.b):
            for h in range(c.Hkv):
                pages = sel[r, h, :cnt[r, h]]
                last = npg[r, h] - 1
                full = int((pages != last).sum())
                toks += full * c.P + (int(n[r, h] - last * c.P) if (pages == last).any() else 0)
        units = int(cnt.sum())
    else:
        toks = int(n.sum())
        units = int(npg.sum())
    kv = toks * 2 * c.d * s
    meta = int(npg.sum()) * 2 * c.d * s if c.topk else 0
    # partials: one row per (r, query head, split touching its head); bounded by
    # (splits + heads per group) * Gq per (r, group)
    rows = c.b * (int(step.S[l].sum()) + c.Hkv) * c.Gq
    small = (c.b * c.Hq * c.d * s * (2 if c.topk else 1)
             + (c.b * c.Hkv * step.layouts[l].page_table.shape[2] * 4 * 2 if c.topk else 0)
             + (c.b * c.Hkv * c.topk * 4 * 2 if c.topk else 0)
             + rows * (c.d + 1) * 4 * 2
             + c.b * c.Hq * c.d * 4)
    maxpg = step.layouts[l].page_table.shape[2]
    return {"kv": kv, "meta": meta, "small": small, "tokens": toks, "units": units,
            "decode_launch": kv + rows * (c.d + 1) * 4 * 2 + c.b * c.Hq * c.d * (s + 4),
            # its two kernels: the split-K decode (KV and q read, partials
            # written) and the combine (partials read, output written)
            "splits_launch": kv + rows * (c.d + 1) * 4 + c.b * c.Hq * c.d * s,
            "combine_launch": rows * (c.d + 1) * 4 + c.b * c.Hq * c.d * 4,
            # per-call bytes of the other rows
            "score_launch": meta + c.b * c.Hq * c.d * s + c.b * c.Hkv * maxpg * 4,
            "topk_launch": int(npg.sum()) * 4 + c.b * c.Hkv * (c.topk or 0) * 4 + c.b * c.Hkv * 4,
            "minmax_launch": int(n.sum()) * c.d * s + int(npg.sum()) * 2 * c.d * s}


def stored_traffic(workload: str):
    """HBM bytes per split-K decode kernel launch from the committed
    rocprofv3 PMC record of this workload (FETCH_SIZE and WRITE_SIZE, scaled
    by a copy of known size), or None if there is none or the decode source
    changed since."""
    from non_uniform_sparse_amd import profiling
    path = os.path.join(ROOT, "profiles", f"decode_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != profiling.decode_source_hash():
        return None
    return rec["traffic_bytes_per_launch"]


def cpu_baseline(wl, step, budget_s: float = 12.0) -> dict:
    """The fp64 oracle timed on this host on a bounded sample of the same
    workload: whole heads (score + top-K + attention; min-max metadata
    precomputed, as on the GPU), until ~budget_s of work."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    # BLAS may use every host core this process is allowed to run on; that
    # count is what the record states.
    cores = len(os.sched_getaffinity(0))
    limiter = threadpool_limits(limits=cores)
    c = wl.cfg
    q = {}
    scale = 1.0 / math.sqrt(c.d)
    done_bytes, spent, heads = 0, 0.0, 0
    order = [(r, l, h) for l in range(c.L) for r in range(c.b) for h in range(c.Hkv)]
    # a workload the oracle finishes quickly is passed over again until the
    # budget is spent, so the figure is not one short, noisy timing
    passes = max(1, int(budget_s / 0.05))
    order = (order * passes)[:max(len(order), 200000)]
    kv_cache = {}
    keep = int(wl.n.sum()) * c.d * 16 <= 2e9     # the fp64 K and V of every head fit in 2 GB
    for r, l, h in order:
        if l not in q:
            q[l] = wl.q(l, device=step.device).double().cpu().numpy()
        pos = int(step.head_slot[l, h])
        if (r, l, h) in kv_cache:
            K, V, lo, hi = kv_cache[(r, l, h)]
        else:
            K, V = wl.head_kv(r, l, h, pos, device=step.device)
            K, V = K.double().cpu().numpy(), V.double().cpu().numpy()
            lo, hi = O.page_minmax(K, c.P)
            if keep:                # a small workload: keep its heads for the next pass
                kv_cache[(r, l, h)] = (K, V, lo, hi)
        qg = q[l][r, h * c.Gq:(h + 1) * c.Gq]
        t0 = time.perf_counter()
        if c.topk:
            pages = O.topk_pages(O.page_scores(qg, lo, hi), c.topk)
        else:
            pages = np.arange(lo.shape[0])
        O.decode_head(qg, K, V, pages, c.P, scale)
        spent += time.perf_counter() - t0
        n = K.shape[0]
        toks = sum(min(c.P, n - int(p) * c.P) for p in pages)
        done_bytes += toks * 2 * c.d * 2
        heads += 1
        if spent >= budget_s:
            break
    limiter.restore_original_limits()
    return {"value": done_bytes / spent / 1e9, "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{heads} whole heads (request-major from layer 0, the workload passed "
                      f"over again while time was left) of {c.name}, "
                      f"{done_bytes / 1e6:.1f} MB of KV in {spent:.1f} s; BLAS threads = "
                      f"cores = {cores} (the host's affinity set); the oracle's loop over "
                      "heads and pages is itself sequential"}


def rerank_reuse_report(configs, period: int = 16, unstable_frac: float = 0.25,
                        reps: int = 10) -> dict:
    """Decoding over steps with stability-aware reranking against reranking
    every head every step (FlexiCache summary, Method; the summary's decode
    microbenchmark compares the two).  Both variants run the same window of
    ``period`` steps -- append, [score + top-K], decode -- captured as one
    graph and replayed from the same starting state; a window costs one
    full rerank plus period - 1 steps in which only unstable heads re-select.
    Windows of small working sets are preceded by a 1 GiB read, as in the
    headline protocol."""
    from non_uniform_sparse_amd.steps import DecodeLoop
    out = {}
    for name in configs:
        ov = {"L": 8} if name == "gemma3_mixed" else {}
        wl = make_workload(name, **ov)
        loop = DecodeLoop(wl, period, device="cuda", period=period, unstable_frac=unstable_frac,
                          poison=False)
        c = wl.cfg
        npg = -(-wl.n // c.P)                                   # [b][L][Hkv]
        small = (np.minimum(npg, c.topk).sum() * 2 * c.P + npg.sum() * 2) * c.d * 2 < 8e9
        flush = torch.ones(1 << 27, dtype=torch.int64, device="cuda") if small else None
        res = {}
        for mode, reuse in (("reuse", True), ("every_step", False)):
            g = loop.capture(period, reuse=reuse)
            times = []
            for _ in range(reps + 2):
                loop.rewind()
                if flush is not None:
                    flush.sum()
                a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b_.record()
                b_.synchronize()
                times.append(a.elapsed_time(b_) / period * 1e3)
            res[mode] = statistics.median(times[2:])
            del g
        unstable = int((~loop.stable).sum())
        out[name] = {
            "layers": c.L, "requests": c.b, "topk_pages": c.topk, "period": period,
            "unstable_heads": f"{unstable} of {c.L * c.Hkv}",
            "all_stable_layers": int(loop.stable.all(axis=1).sum()),
            "us_per_step_reuse": round(res["reuse"], 1),
            "us_per_step_every_step": round(res["every_step"], 1),
            "speedup": round(res["every_step"] / res["reuse"], 3),
            "includes": "append + scoring/top-K of the heads due + decode, per step",
        }
        del loop
        torch.cuda.empty_cache()
    return out


def sparse_dense_report(configs, reps: int = 20) -> dict:
    """Top-K sparse decode against dense decode on the same caches (FlexiCache
    summary, Experiments: the decode microbenchmark compares the two).  The
    sparse step is score + top-K + decode over the selected pages; the dense
    step decodes every retained page with its own split plan (no top-K cap
    on the budgets).  Both are captured as graphs (request micro-batches as
    the headline uses them) and replayed; small working sets are preceded by
    a 1 GiB read, as in the headline protocol."""
    out = {}
    for name in configs:
        ov = {"L": 8} if name == "gemma3_mixed" else {}
        res, kv_bytes = {}, {}
        for mode in ("sparse", "dense"):
            wl = make_workload(name, **ov) if mode == "sparse" else \
                make_workload(name, topk=None, **ov)
            c = wl.cfg
            step = DecodeStep(wl, device="cuda", poison=False,
                              microbatches=default_microbatches(wl))
            qs = step.queries()
            g = step.capture(qs)               # runs the step once eagerly first
            torch.cuda.synchronize()
            kv_bytes[mode] = sum(algorithmic_bytes(step, l)["kv"] for l in range(c.L))
            flush = torch.ones(1 << 27, dtype=torch.int64, device="cuda") \
                if kv_bytes[mode] < 8e9 else None
            times = []
            for _ in range(reps + 2):
                if flush is not None:
                    flush.sum()
                a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b_.record()
                b_.synchronize()
                times.append(a.elapsed_time(b_) * 1e3)
            res[mode] = statistics.median(times[2:])
            del g, step, flush
            torch.cuda.empty_cache()
        out[name] = {
            "layers": c.L, "requests": c.b, "topk_pages": CONFIGS[name].topk,
            "us_per_step_sparse": round(res["sparse"], 1),
            "us_per_step_dense": round(res["dense"], 1),
            "speedup": round(res["dense"] / res["sparse"], 3),
            "kv_bytes_sparse": int(kv_bytes["sparse"]), "kv_bytes_dense": int(kv_bytes["dense"]),
            "dense_kv_GBps": round(kv_bytes["dense"] / (res["dense"] * 1e-6) / 1e9, 1),
            "includes": "sparse: scoring + top-K + decode; dense: decode of every retained page",
        }
    return out


def prefill_report(configs, chunk: int = 2048) -> dict:
    """Chunked prefill under Budget Reservation (Tangram review, 3.1): every
    chunk of every layer, selection + compaction + page bounds in one
    kvs_prefill_chunk launch each.  Each launch is timed with events behind a
    short GPU spin (its inputs are generated before and are not timed).
    Bytes: the chunk's scores, the kept tokens' K/V read and written, and
    the bounds of the pages written."""
    from non_uniform_sparse_amd.prefill import ChunkedPrefill
    out = {}
    stream = torch.cuda.current_stream()
    rate = sleep_rate(stream)
    for name in configs:
        ov = {"L": 8} if name == "gemma3_mixed" else {}
        wl = make_workload(name, **ov)
        c = wl.cfg
        pf = ChunkedPrefill(wl, chunk, device="cuda")
        total_ms, total_bytes, kept, launches = 0.0, 0, 0, 0
        for k in range(pf.chunks):
            for l in range(c.L):
                inp = pf.inputs(l, k)
                q_np = pf.quota(l, k)
                q = torch.from_numpy(q_np).to("cuda")
                torch.cuda._sleep(int(rate * 0.3))
                a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                pf.run_chunk(l, k, inputs=inp, quota=q)
                b_.record()
                b_.synchronize()
                total_ms += a.elapsed_time(b_)
                qs = int(q_np.sum())
                pages = int(np.ceil(q_np / c.P).sum()) + c.b * c.Hkv   # bound on pages touched
                total_bytes += (c.b * c.Hkv * chunk * 4 + qs * 2 * c.d * 2 * 2
                                + pages * 2 * c.d * 2)
                kept += qs
                launches += 1
        gbps = total_bytes / (total_ms * 1e-3) / 1e9
        out[name] = {"layers": c.L, "requests": c.b, "chunk": chunk, "launches": launches,
                     "tokens_in": int(wl.contexts.sum()) * c.L * c.Hkv, "tokens_kept": kept,
                     "us_per_launch": round(total_ms / launches * 1e3, 2),
                     "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}
        del pf
        torch.cuda.empty_cache()
    return out


def tier_report(name: str = "flexicache_topk", period: int = 16, windows: int = 3,
                unstable_frac: float = 0.25) -> dict:
    """Tiered placement of stable heads (FlexiCache summary, tiered
    placement), one page table per head.  Times, with events behind a short
    GPU spin: the bulk offload of the stable heads' pages after prefill
    (GPU -> pinned host), the promotion after each rerank (host -> GPU, only
    newly selected pages), and whole rerank windows of ``period`` steps on
    the tiered and on the fully resident cache.  The host-link figures are
    set against a plain pinned-to-device copy of 256 MiB measured here."""
    from non_uniform_sparse_amd.tiered import TieredLoop
    from non_uniform_sparse_amd.kvs import Tier
    stream = torch.cuda.current_stream()
    rate = sleep_rate(stream)

    def timed(fn, spin_ms=0.3):
        torch.cuda._sleep(int(rate * spin_ms))
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b_.record()
        b_.synchronize()
        return a.elapsed_time(b_)

    # plain copies over the host link, both directions
    n = 256 << 20
    h = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    h.fill_(1)
    dbuf = torch.empty(n, dtype=torch.uint8, device="cuda")
    h2d = min(timed(lambda: dbuf.copy_(h, non_blocking=True)) for _ in range(5))
    d2h = min(timed(lambda: h.copy_(dbuf, non_blocking=True)) for _ in range(5))
    del h, dbuf
    copy_h2d, copy_d2h = n / (h2d * 1e-3) / 1e9, n / (d2h * 1e-3) / 1e9

    wl = make_workload(name, Hp=1)
    c = wl.cfg
    steps = period * windows + 1
    page_bytes = 2 * c.P * c.d * 2
    # bulk offload, timed on a fully resident cache of its own
    full = DecodeStep(wl, device="cuda", poison=False)
    stable = wl.stable_heads(unstable_frac)
    npg = -(-wl.n // c.P)                                         # [b][L][Hkv]
    off_ms, off_pages = 0.0, 0
    for l in range(c.L):
        hb = np.full((c.b, c.Hkv), -1, dtype=np.int64)
        run = 0
        for r in range(c.b):
            for hh in range(c.Hkv):
                if stable[l, hh]:
                    hb[r, hh] = run
                    run += int(npg[r, l, hh])
        host = torch.empty((max(1, run), 2, c.P, c.d), dtype=full.caches[l].kv.dtype,
                           pin_memory=True)
        dummy = torch.full((c.b, c.Hkv, 1), -1, dtype=torch.int32, device="cuda")
        tier = Tier(host, torch.from_numpy(hb).to("cuda"), dummy, dummy)
        off_ms += timed(lambda: kvs.kvs_offload_pages(full.caches[l], tier))
        off_pages += run
        del host
    del full
    torch.cuda.empty_cache()

    res = {}
    for mode in ("tiered", "resident", "tiered_append", "resident_append"):
        loop = TieredLoop(wl, steps, period=period, tiered=mode.startswith("tiered"),
                          stable=stable, append=mode.endswith("append"))
        if mode == "tiered":
            gpu_b, full_b = loop.gpu_bytes, loop.full_bytes
        prom = []
        for t in range(steps):
            if mode.startswith("tiered") and t % period == 0:
                if loop.append:
                    for l in range(c.L):
                        k, v = loop.kv[t][l]
                        kvs.kvs_append_kv_tier(loop.ds.caches[l], loop.tiers[l], k, v)
                due = [loop.select(t, l) for l in range(c.L)]
                torch.cuda.synchronize()
                ms = timed(lambda: [loop.promote(l, due[l]) for l in range(c.L)])
                moved = sum(int(m.sum().item()) for m in loop.moved)
                prom.append((t, ms, moved))
                for l in range(c.L):
                    loop.ds.attend(l, loop.q[t][l])
            else:
                loop.run_step(t)
        torch.cuda.synchronize()
        # whole windows from the start, replayed as one graph
        g = loop.capture(steps - 1)
        wms = []
        for _ in range(4):
            loop.rewind()
            torch.cuda.synchronize()
            wms.append(timed(g.replay, spin_ms=1.0))
        res[mode] = {"us_per_step": statistics.median(wms[1:]) / (steps - 1) * 1e3, "prom": prom}
        del g, loop
        torch.cuda.empty_cache()
    stable_heads = c.b * int(stable.sum())
    reranks = [{"step": t, "pages_moved": m,
                "frac_of_topk": round(m / (stable_heads * c.topk), 3),
                "us": round(ms * 1e3, 1),
                "GBps": round(m * page_bytes / (ms * 1e-3) / 1e9, 2)}
               for t, ms, m in res["tiered"]["prom"]]
    later = [r for r in reranks if r["step"] > 0]
    return {
        "config": {"workload": name, "requests": c.b, "layers": c.L, "kv_heads": c.Hkv,
                   "tokens": c.N, "topk_pages": c.topk, "page_bytes": page_bytes,
                   "heads_per_page_table": 1, "period": period,
                   "stable_heads": f"{int(stable.sum())} of {c.L * c.Hkv} per request"},
        "gpu_kv_bytes": {"tiered": gpu_b, "resident": full_b,
                         "saved": round(1 - gpu_b / full_b, 3)},
        "host_link": {"copy_h2d_GBps": round(copy_h2d, 1), "copy_d2h_GBps": round(copy_d2h, 1),
                      "nominal_GBps": 64.0, "note": "PCIe 5.0 x16, one direction"},
        "offload": {"pages": off_pages, "us": round(off_ms * 1e3, 1),
                    "GBps": round(off_pages * page_bytes / (off_ms * 1e-3) / 1e9, 2)},
        "promotion": reranks,
        "promotion_later_reranks_GBps": round(statistics.mean([r["GBps"] for r in later]), 2)
        if later else None,
        "us_per_step": {m: round(res[m]["us_per_step"], 1) for m in res},
        "window": f"steps 0..{steps - 2} as one graph: {windows} reranks with promotion, the "
                  "other steps scoring only unstable heads; *_append: each step first appends "
                  "its token (written through to the host pages when tiered)",
    }


def codec_report(name: str = "llama7b_chunk", reps: int = 10) -> dict:
    """KV-cache codec after CacheGen (paper notes, sections 3 and 7): one
    chunk encoded on the host, then decoded on the GPU.  The decode is timed
    with events behind a short GPU spin (median of ``reps``); the encoded
    chunk and, for comparison, the raw fp16 chunk are timed as single pinned
    host-to-device copies -- the transfer the codec shrinks."""
    from non_uniform_sparse_amd import codec
    cfg = codec.CHUNKS[name]
    x = codec.make_chunk(cfg)
    lay = codec.layout_of(cfg)
    t0 = time.perf_counter()
    enc = kvs.kvs_codec_encode(lay, x)
    enc_s = time.perf_counter() - t0
    d = enc.to("cuda")
    out = torch.empty((cfg.L, 2, cfg.T, cfg.C), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()
    rate = sleep_rate(stream)
    kvs.kvs_codec_decode(d, out)
    times = []
    for _ in range(reps):
        torch.cuda._sleep(int(rate * 0.5))
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        kvs.kvs_codec_decode(d, out)
        b_.record()
        b_.synchronize()
        times.append(a.elapsed_time(b_))
    ms = statistics.median(times)
    raw = x.numel() * 2
    coded = enc.nbytes()

    def h2d_ms(nbytes):
        h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        dd = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        best = float("inf")
        for _ in range(3):
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dd.copy_(h, non_blocking=True)
            b_.record()
            b_.synchronize()
            best = min(best, a.elapsed_time(b_))
        return best

    # pipelined loading (transfer of chunk i overlapping the decode of chunk
    # i - 1): the chunk, pinned once, loaded 4 times into two alternating outputs
    pinned = codec.pin(enc)
    loader = codec.PipelinedLoader(lay, enc.cdf.numel(), enc.streams.numel())
    outs = [out, torch.empty_like(out)]
    n_chunks = 4
    loader.run([pinned] * 2, outs)
    torch.cuda.synchronize()
    a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    loader.run([pinned] * n_chunks, [outs[i % 2] for i in range(n_chunks)])
    b_.record()
    b_.synchronize()
    pipe_ms = a.elapsed_time(b_) / n_chunks
    symbols = cfg.L * 2 * cfg.T * cfg.C
    return {
        "config": {"workload": name, "layers": cfg.L, "tokens": cfg.T, "channels": cfg.C,
                   "group": cfg.group, "channels_per_stream": cfg.S, "rho": cfg.rho,
                   "streams": cfg.L * 2 * (cfg.C // cfg.S) * cfg.T},
        "raw_bytes": raw, "encoded_bytes": coded, "ratio": round(raw / coded, 3),
        "bits_per_value": round(8 * coded / symbols, 3),
        "encode_host_s": round(enc_s, 3),
        "decode_us": round(ms * 1e3, 1),
        "decode_out_GBps": round(raw / (ms * 1e-3) / 1e9, 1),
        "decode_Gsymbols_per_s": round(symbols / (ms * 1e-3) / 1e9, 1),
        "h2d_encoded_us": round(h2d_ms(coded) * 1e3, 1),
        "h2d_raw_us": round(h2d_ms(raw) * 1e3, 1),
        "pipelined_us_per_chunk": round(pipe_ms * 1e3, 1),
        "pipelined": f"{n_chunks} chunks from pinned host memory, the copy of chunk i "
                     "overlapping the decode of chunk i - 1 (two streams, two buffer sets)",
    }


def skew_report(configs, launches: int = 20, T=None) -> dict:
    """Per-workgroup duration skew of the split-K decode kernel (max / mean
    over the workgroups of one launch, median over launches, per layer) and
    the launch's duration (HIP events, median over launches, per layer), with
    the planned split map and with a uniform one of the same total (equal
    budgets).  The launches of a layer are queued back to back behind a GPU
    spin, each followed by a copy of its stamps.  Uses the stamp-instrumented
    library build (each workgroup records its start and end)."""
    from non_uniform_sparse_amd import build as B
    kvs.use_library(B.LIB_STAMPS)
    out = {}
    for name in configs:
        wl = make_workload(name)
        c = wl.cfg
        step = DecodeStep(wl, device="cuda:0", T=T)
        qs = step.queries()
        if c.topk:
            for l in range(c.L):
                step.select(l, qs[l])
        stream = torch.cuda.Stream()
        rate = sleep_rate(stream)

        def row_of(label, l):
            return step.S[l] if label == "planned" else kvs.kvs_plan_split(
                np.ones((1, c.Hkv)), step.head_slot[l:l + 1], c.Hp, 0.0, int(step.S[l].sum()))[0]
        for label in ("planned", "uniform"):           # warm-up: every layer, both maps
            for l in range(c.L):
                row = row_of(label, l)
                need = kvs.kvs_decode_workspace_bytes(c.b, c.Hq, c.Hkv, c.d, row)
                if need > step.workspace.numel():
                    step.workspace = torch.empty(need, dtype=torch.uint8, device="cuda:0")
                step.attend(l, qs[l], stream, S_row=row)
        stream.synchronize()
        res = {}
        for label in ("planned", "uniform"):
            skew_l, us_l, xcd_l = [], [], []
            for l in range(c.L):
                row = row_of(label, l)
                off = kvs.kvs_decode_stamps_offset(c.b, c.Hq, c.Hkv, c.d, row)
                nwg = c.b * int(np.sum(row))
                src = step.workspace[off:off + nwg * 16].view(torch.int64).view(nwg, 2)
                stamps = torch.empty((launches, nwg, 2), dtype=torch.int64, device="cuda:0")
                marks = []
                with torch.cuda.stream(stream):   # a spin long enough for the host to enqueue
                    torch.cuda._sleep(int(rate * (2.0 + 0.5 * launches)))
                    for i in range(launches):
                        e0, e1 = torch.cuda.Event(enable_timing=True), \
                            torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        step.attend(l, qs[l], stream, S_row=row)
                        e1.record(stream)
                        stamps[i].copy_(src)
                        marks.append((e0, e1))
                stream.synchronize()
                dur = (stamps[:, :, 1] - stamps[:, :, 0]).double().cpu()      # [launch][wg]
                skew_l.append(statistics.median((dur.max(1).values / dur.mean(1)).tolist()))
                us_l.append(statistics.median(a.elapsed_time(b_) * 1e3 for a, b_ in marks))
                # workgroups go round-robin over the 8 XCDs: mean duration per XCD
                xm = dur.view(launches, -1, 8).mean(1) if nwg % 8 == 0 else None
                if xm is not None:
                    xcd_l.append(statistics.median((xm.max(1).values / xm.min(1).values).tolist()))
            worst = int(np.argmax(skew_l))
            res[label] = {
                "skew_median_over_layers": round(statistics.median(skew_l), 3),
                "skew_worst_layer": round(skew_l[worst], 3), "worst_layer": worst,
                "skew_per_layer": [round(x, 3) for x in skew_l],
                "decode_us_per_layer": [round(x, 1) for x in us_l],
                "decode_us_sum": round(sum(us_l), 1),
                "xcd_mean_duration_max_over_min_median": (round(statistics.median(xcd_l), 3)
                                                          if xcd_l else None),
            }
        res["splits_per_request"] = step.T
        res["uniform_over_planned_decode_us"] = round(
            res["uniform"]["decode_us_sum"] / res["planned"]["decode_us_sum"], 3)
        res["note"] = ("skew = max / mean workgroup duration of one launch (s_memrealtime "
                       "stamps), median over launches; decode_us from HIP events around each "
                       "launch of the instrumented build (split kernel + combine)")
        out[name] = res
        del step
        torch.cuda.empty_cache()
    return out


def sleep_rate(stream) -> float:
    """Spin cycles per millisecond of torch's GPU sleep kernel, measured."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 1 << 20
    with torch.cuda.stream(stream):
        torch.cuda._sleep(n)
        a.record(stream)
        torch.cuda._sleep(n)
        b.record(stream)
    b.synchronize()
    return n / max(a.elapsed_time(b), 1e-3)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=sorted(CONFIGS))
    ap.add_argument("--microbatches", type=int, default=0,
                    help="request micro-batches, each on a stream of its own in the step graph "
                         "(0: one below 4 layers, else min(3, requests))")
    ap.add_argument("--fused-select", choices=["auto", "on", "off"], default="auto",
                    help="score + top-K in one launch per layer: auto (layers whose heads are of "
                         "similar length), on, off")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill", nargs="*", default=None, metavar="CONFIG",
                    help="time the chunked prefill under Budget Reservation (default configs: "
                         "llama8b_ragged, gemma3_mixed at 8 layers) and print that record")
    ap.add_argument("--rerank-reuse", nargs="*", default=None, metavar="CONFIG",
                    help="time decoding over steps with stability-aware reranking against "
                         "reranking every step (default configs: flexicache_topk, gemma3_mixed "
                         "at 8 layers) and print that record instead of the step line")
    ap.add_argument("--tier", nargs="?", const="flexicache_topk", default=None, metavar="CONFIG",
                    help="time tiered placement of stable heads (offload, promotion over the "
                         "host link, rerank windows tiered vs resident), print it and exit")
    ap.add_argument("--codec", nargs="?", const="llama7b_chunk", default=None, metavar="CHUNK",
                    help="encode a KV chunk on the host and time its GPU decode, print it "
                         "and exit")
    ap.add_argument("--sparse-vs-dense", nargs="*", default=None, metavar="CONFIG",
                    help="time the top-K sparse step against dense decode on the same caches "
                         "(default configs: flexicache_topk, gemma3_mixed at 8 layers), print "
                         "that record and exit")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--logits", choices=["mfma", "valu"], default="mfma",
                    help="decode logits on MFMA (the library) or on the VALU (the measurement "
                         "build that backs the MFMA choice)")
    ap.add_argument("--splits", type=int, default=None,
                    help="splits per request per layer (default: the planned rule)")
    ap.add_argument("--skew", nargs="*", default=None, metavar="CONFIG",
                    help="measure per-workgroup duration skew (planned vs uniform split "
                         "map) with the instrumented build, print it and exit")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 1 GiB device copy (known bytes) to scale "
                         "hardware byte counters, then exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path here runs on a single MI355X; "
              "run with --gpus 1", file=sys.stderr)
        return 2
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.logits == "valu":
        from non_uniform_sparse_amd import build as B
        kvs.use_library(B.LIB_VALU)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.prefill is not None:
        print(json.dumps({"prefill": prefill_report(args.prefill or ["llama8b_ragged",
                                                                     "gemma3_mixed"])}))
        return 0
    if args.rerank_reuse is not None:
        print(json.dumps({"rerank_reuse": rerank_reuse_report(
            args.rerank_reuse or ["flexicache_topk", "gemma3_mixed"])}))
        return 0
    if args.codec is not None:
        print(json.dumps({"codec": codec_report(args.codec)}))
        return 0
    if args.sparse_vs_dense is not None:
        print(json.dumps({"sparse_vs_dense": sparse_dense_report(
            args.sparse_vs_dense or ["flexicache_topk", "gemma3_mixed"])}))
        return 0
    if args.tier is not None:
        print(json.dumps({"tier": tier_report(args.tier)}))
        return 0
    if args.skew is not None:
        print(json.dumps({"skew": skew_report(args.skew or ["llama8b_ragged", "longctx_skew"],
                                              T=args.splits)}))
        return 0
    if args.copy_probe:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(5):
            a.record()
            dst.copy_(src)
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b))
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                          "ms": round(min(times), 4),
                          "GBps_read_plus_write": round(2 * n / (min(times) * 1e-3) / 1e9, 1)}))
        return 0

    t0 = time.time()
    wl = make_workload(args.config)
    c = wl.cfg
    step = DecodeStep(wl, device=dev, T=args.splits,
                      microbatches=args.microbatches or default_microbatches(wl),
                      fused={"auto": None, "on": True, "off": False}[args.fused_select])
    qs = step.queries()
    torch.cuda.synchronize()
    log(f"[bench] {c.name}: set-up {time.time() - t0:.1f} s, W={step.W}, T={step.T}, "
        f"S[0]={step.S[0].tolist()}")

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step.run(qs, stream)
    stream.synchronize()
    ab = [algorithmic_bytes(step, l) for l in range(c.L)]
    kv_bytes = sum(a["kv"] for a in ab)
    path_bytes = sum(a["kv"] + a["meta"] + a["small"] for a in ab)
    # Working sets that could sit in L2 / MALL (256 MB) are evicted before
    # each step by reading 1 GB (a read leaves no dirty lines behind to be
    # written back inside the timed step).
    flush = torch.ones(1 << 27, dtype=torch.int64, device=dev) if path_bytes < 8e9 else None
    ev = lambda: torch.cuda.Event(enable_timing=True)
    cycles_per_ms = sleep_rate(stream)

    # Pass 1 (eager, per-kernel HIP events on the launch stream): kernel
    # durations for the roofline figures.  Each step is queued behind a GPU
    # spin long enough for the host to enqueue the whole step, so the
    # kernels run back to back and the events time kernels, not host
    # launch latency.
    kern = {"score": [], "topk": [], "select": [], "decode_splits": [], "decode_combine": [],
            "decode_attn": []}
    for _ in range(args.steps):
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(cycles_per_ms * (2.0 + 0.4 * c.L)))
            if flush is not None:
                flush.sum()
        marks = []
        for l in range(c.L):
            q = qs[l]
            if c.topk and step.fused[l]:
                a, b_ = ev(), ev()
                a.record(stream)
                kvs.kvs_select_pages(step.caches[l], q, step.bufs[l].scores, c.topk,
                                     step.bufs[l].sel, step.bufs[l].sel_count, stream)
                b_.record(stream)
                marks.append(("select", a, b_))
            elif c.topk:
                a, b_, d_ = ev(), ev(), ev()
                a.record(stream)
                kvs.kvs_score_pages(step.caches[l], q, step.bufs[l].scores, stream)
                b_.record(stream)
                kvs.kvs_topk_pages(step.bufs[l].scores, step.caches[l].seq_len, c.P, c.topk,
                                   step.bufs[l].sel, step.bufs[l].sel_count, stream)
                d_.record(stream)
                marks.append(("score", a, b_))
                marks.append(("topk", b_, d_))
            e0, e1 = ev(), ev()
            e0.record(stream)
            step.attend(l, q, stream)
            e1.record(stream)
            marks.append(("decode_attn", e0, e1))
        stream.synchronize()
        for k, a, b_ in marks:
            kern[k].append(a.elapsed_time(b_))
        # the decode's two kernels again, as the two calls kvs_decode_splits
        # and kvs_decode_combine (the same kernels as one kvs_decode_attn),
        # each timed alone
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(cycles_per_ms * (1.0 + 0.2 * c.L)))
            if flush is not None:
                flush.sum()
        marks = []
        for l in range(c.L):
            buf = step.bufs[l]
            dargs = (step.caches[l], qs[l], buf.sel, buf.sel_count, c.topk or 0, step.S[l],
                     step.scale, step.workspace, buf.out, stream)
            e0, e1, e2 = ev(), ev(), ev()
            e0.record(stream)
            kvs.kvs_decode_splits(*dargs)
            e1.record(stream)
            kvs.kvs_decode_combine(*dargs)
            e2.record(stream)
            marks.append(("decode_splits", e0, e1))
            marks.append(("decode_combine", e1, e2))
        stream.synchronize()
        for k, a, b_ in marks:
            kern[k].append(a.elapsed_time(b_))

    # Pass 2 (headline): the whole step captured once as a HIP graph (the
    # request micro-batches on streams of their own) and replayed; K steps
    # timed between two synchronisations.
    graph = step.capture(qs)
    cur = torch.cuda.current_stream()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    marks = []
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        if flush is not None:
            flush.sum()
        s0, s1 = ev(), ev()
        s0.record(cur)
        graph.replay()
        s1.record(cur)
        marks.append((s0, s1))
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3

    # With flushes the steps are timed one by one (the flush is not step
    # work); without, the wall clock over the K back-to-back replays.  The
    # per-step events give the spread either way.
    per_step = sorted(a.elapsed_time(b_) for a, b_ in marks)
    ms = statistics.mean(per_step) if flush is not None else wall_ms / args.steps

    # The other rows of the path, each against the HBM peak: the min-max build
    # (once per page fill, not in the step) re-run per layer behind a GPU spin,
    # and the host planner.
    mm_ms = []
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(cycles_per_ms * (2.0 + 0.1 * c.L)))
        mm_marks = []
        for l in range(c.L):
            a, b_ = ev(), ev()
            a.record(stream)
            kvs.kvs_build_minmax(step.caches[l], stream)
            b_.record(stream)
            mm_marks.append((a, b_))
    stream.synchronize()
    mm_ms = [a.elapsed_time(b_) for a, b_ in mm_marks]
    # The empirical ceiling of the decode's gather: the same K/V tiles of the
    # attended pages read through the page table with no arithmetic
    # (kvs_gather_probe), per layer behind a GPU spin.
    sink = torch.empty(kvs.kvs_gather_probe_sink_words(c.d), dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(cycles_per_ms * (2.0 + 0.1 * c.L)))
        pr_marks = []
        for l in range(c.L):
            a, b_ = ev(), ev()
            buf = step.bufs[l]
            a.record(stream)
            kvs.kvs_gather_probe(step.caches[l], buf.sel if c.topk else None,
                                 buf.sel_count if c.topk else None, c.topk or 0, sink, stream)
            b_.record(stream)
            pr_marks.append((a, b_))
    stream.synchronize()
    pr_ms = statistics.mean(a.elapsed_time(b_) for a, b_ in pr_marks)
    units = [int(step.bufs[l].sel_count.sum()) if c.topk else int((-(-wl.n[:, l, :] // c.P)).sum())
             for l in range(c.L)]
    pr_bytes = statistics.mean(units) * 2 * c.P * c.d * 2
    pr_gbps = pr_bytes / (pr_ms * 1e-3) / 1e9
    # Plain contiguous reads of the kernels' own byte counts (no gather, no
    # arithmetic): the chip's rate for a launch of that size.  Successive
    # launches read successive windows of a 4 GiB buffer, so none is served
    # by the caches.
    region = torch.empty(1 << 30, dtype=torch.int32, device=dev)
    sp_sink = torch.empty(kvs.kvs_stream_probe_sink_words(), dtype=torch.int32, device=dev)

    def stream_us(nbytes: int, reps: int = 12) -> float:
        nbytes = min((int(nbytes) + 15) // 16 * 16, region.numel() * 4 // 2)
        wins = region.numel() * 4 // nbytes
        marks = []
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(cycles_per_ms * 2.0))
            for i in range(reps):
                win = region.view(torch.uint8)[(i % wins) * nbytes:]
                a, b_ = ev(), ev()
                a.record(stream)
                kvs.kvs_stream_probe(win, nbytes, sp_sink, stream)
                b_.record(stream)
                marks.append((a, b_))
        stream.synchronize()
        return statistics.mean(a.elapsed_time(b_) for a, b_ in marks[2:]) * 1e3
    plain = {"decode": statistics.mean(a["splits_launch"] for a in ab)}
    if c.topk:
        plain["score"] = statistics.mean(a["score_launch"] for a in ab)
    plain_rows = {}
    for k, nb in plain.items():
        us = stream_us(nb)
        plain_rows[f"plain_read_{k}_bytes"] = {
            "us": round(us, 2), "bytes": int(nb), "GBps": round(nb / (us * 1e-6) / 1e9, 1),
            "frac": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": f"a plain contiguous read of the {k} launch's byte count (kvs_stream_probe)"}
    del region
    t_plan = time.perf_counter()
    for _ in range(20):
        kvs.kvs_plan_split(wl.budgets, step.head_slot, c.Hp, 0.0, step.T)
    plan_us = (time.perf_counter() - t_plan) / 20 * 1e6

    def row(ms_list, key):
        t = statistics.mean(ms_list)
        by = statistics.mean(a[key] for a in ab)
        gbps = by / (t * 1e-3) / 1e9
        return {"us": round(t * 1e3, 2), "bytes": int(by), "GBps": round(gbps, 1),
                "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    rows = {"a1_minmax_build": dict(row(mm_ms, "minmax_launch"),
                                    note="once per page fill, not part of the step")}
    if kern["score"]:
        rows["a2_score"] = row(kern["score"], "score_launch")
        rows["a3_topk"] = dict(row(kern["topk"], "topk_launch"), bound="latency")
    if kern["select"]:
        rows["a2_a3_select"] = dict(row(kern["select"], "score_launch"),
                                    note="scores and top-K in one launch (kvs_select_pages); "
                                         "bytes are the scoring's")
    rows["a4_plan"] = {"us_host": round(plan_us, 1), "note": f"S[{c.L}][{c.G}], host, ahead of time"}
    rows["a5_decode_splits"] = dict(row(kern["decode_splits"], "splits_launch"),
                                    note="the split-K decode kernel alone (kvs_decode_splits)")
    rows["a6_combine"] = dict(row(kern["decode_combine"], "combine_launch"),
                              note="the LSE combine kernel alone (kvs_decode_combine)")
    rows["a5_a6_decode_combine"] = dict(row(kern["decode_attn"], "decode_launch"),
                                        note="one kvs_decode_attn call: both kernels and the "
                                             "gap between them")
    rows.update(plain_rows)
    rows["gather_probe"] = {"us": round(pr_ms * 1e3, 2), "bytes": int(pr_bytes),
                            "GBps": round(pr_gbps, 1), "frac": round(pr_gbps / HBM_PEAK_GBPS, 4),
                            "note": "the decode's K/V tiles read through the page table, no "
                                    "arithmetic: the access pattern's empirical ceiling"}
    pct = lambda f: per_step[min(len(per_step) - 1, int(f * len(per_step)))]
    # The dominant kernel: the split-K decode, timed alone.
    dec_ms = statistics.mean(kern["decode_splits"])
    dec_bytes = statistics.mean(a["splits_launch"] for a in ab)
    achieved = dec_bytes / (dec_ms * 1e-3) / 1e9
    value = kv_bytes / (ms * 1e-3) / 1e9
    traffic = stored_traffic(c.name)
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "us_per_step": round(ms * 1e3, 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "path_GBps": round(path_bytes / (ms * 1e-3) / 1e9, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {
            "workload": c.name, "requests": c.b, "layers": c.L, "q_heads": c.Hq,
            "kv_heads": c.Hkv, "head_dim": c.d, "page": c.P, "Hp": c.Hp,
            "topk_pages": c.topk, "splits_per_request": step.T,
            "kv_bytes_per_step": kv_bytes, "path_bytes_per_step": path_bytes,
            "cache_flush_between_steps": flush is not None,
            "step_launch": "hip_graph",
            "microbatches": len(step.parts),
            "fused_select_layers": int(sum(step.fused)),
        },
        "kernels_ms_avg": {k: round(statistics.mean(v), 5) for k, v in kern.items() if v},
        "rows": rows,
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_kernel (the split-K decode, kvs_decode_splits)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "empirical_ceiling_GBps": round(pr_gbps, 1),
            "frac_of_empirical_ceiling": round(achieved / pr_gbps, 4),
            "plain_read_same_bytes_GBps": plain_rows["plain_read_decode_bytes"]["GBps"],
            "with_combine_frac": rows["a5_a6_decode_combine"]["frac"],
        },
        "wall_ms_per_step_incl_flush": round(wall_ms / args.steps, 4),
        "step_ms_p10_p50_p90": [round(pct(0.1), 4), round(statistics.median(per_step), 4),
                                round(pct(0.9), 4)],
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host ...")
        rec["cpu_baseline"] = cpu_baseline(wl, step, args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
