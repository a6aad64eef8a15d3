"""kvs_decode_attn_noalloc, the decode entry point that allocates nothing
(its workspace is the library's own per-device scratch array), against
kvs_decode_attn with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller input, each output equal bit for bit (the same
kernels on the same inputs), so the oracle bar the decode meets carries
over."""

import numpy as np
import pytest
import torch

from gpu_harness import require_gpu, say
from non_uniform_sparse_amd import kvs
from non_uniform_sparse_amd.pipeline import DecodeStep
from non_uniform_sparse_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def _both(step):
    c = step.cfg
    q = step.queries()[0]
    if c.topk:
        step.select(0, q)
    buf = step.bufs[0]
    sel = buf.sel if c.topk else None
    cnt = buf.sel_count if c.topk else None
    ref = torch.full((c.b, c.Hq, c.d), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full_like(ref, float("nan"))
    kvs.kvs_decode_attn(step.caches[0], q, sel, cnt, c.topk or 0, step.S[0], step.scale,
                        step.workspace, ref)
    kvs.kvs_decode_attn_noalloc(step.caches[0], q, sel, cnt, c.topk or 0, step.S[0], step.scale,
                                got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_entry():
    require_gpu()
    cases = [("flexicache_topk", dict(b=6, N=3000)),              # larger first
             ("llama8b_ragged", dict(b=2, N=900, d=256, Hq=16))]  # then a smaller one
    for name, ov in cases:
        say(f"[case] noalloc {name} {ov}")
        wl = make_workload(name, **ov)
        step = DecodeStep(wl, device="cuda")
        need = kvs.kvs_decode_workspace_bytes(wl.cfg.b, wl.cfg.Hq, wl.cfg.Hkv, wl.cfg.d,
                                              step.S[0])
        assert need <= kvs.NOALLOC_SCRATCH_BYTES
        ref, got = _both(step)
        assert torch.isfinite(ref).all()
        assert torch.equal(got, ref), f"{name}: max diff {(got - ref).abs().max().item()}"
        say(f"{name}: outputs equal ({ref.numel()} values, workspace {need} bytes)")


def test_noalloc_rejects_oversized_shape():
    """A split row whose workspace exceeds the scratch is refused, nothing runs."""
    require_gpu()
    wl = make_workload("llama8b_ragged", b=2, N=900)
    step = DecodeStep(wl, device="cuda")
    c = wl.cfg
    q = step.queries()[0]
    out = torch.zeros((c.b, c.Hq, c.d), dtype=torch.float32, device="cuda")
    row = np.full(c.G, 30000, dtype=np.int32)   # within the 65536-split cap
    assert kvs.kvs_decode_workspace_bytes(c.b, c.Hq, c.Hkv, c.d, row) > kvs.NOALLOC_SCRATCH_BYTES
    with pytest.raises(kvs.KvsError) as e:
        kvs.kvs_decode_attn_noalloc(step.caches[0], q, None, None, 0, row, step.scale, out)
    assert e.value.code == kvs.KVS_ENOSPC
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
