"""The gather probe (the decode's access pattern read with no arithmetic,
the bench's empirical ceiling) reads exactly the attended tiles: the XOR of
its sink equals the XOR of every 32-bit word of the K/V tiles of the pages
the decode attends, gathered on the host side through the page table; null
pages count for nothing."""

import numpy as np
import pytest
import torch

from gpu_harness import require_gpu, say
from non_uniform_sparse_amd import kvs
from non_uniform_sparse_amd.pipeline import DecodeStep
from non_uniform_sparse_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def _want(cache, sel, cnt, P):
    kv = cache.kv.view(torch.int32).cpu().numpy()          # [pages][Hp][2*P*d/2]
    kv = kv.reshape(kv.shape[0], kv.shape[1], -1)
    pt = cache.page_table.cpu().numpy()
    seq = cache.seq_len.cpu().numpy()
    hs = cache.head_slot.cpu().numpy()
    Hp = kv.shape[1]
    acc = np.int32(0)
    b, Hkv = seq.shape
    for r in range(b):
        for h in range(Hkv):
            npg = -(-int(seq[r, h]) // P)
            pages = sel[r, h, :cnt[r, h]] if sel is not None else np.arange(npg)
            for p in pages:
                phys = pt[r, hs[h] // Hp, p]
                if 0 <= phys < kv.shape[0]:
                    acc ^= np.bitwise_xor.reduce(kv[phys, hs[h] % Hp])
    return acc


@pytest.mark.parametrize("name,ov,null_pages", [
    ("flexicache_topk", dict(b=3, N=700), False),
    ("flexicache_topk", dict(b=2, N=900), True),
    ("gemma3_mixed", dict(b=3, L=1, N=4096, topk=16), False),
    ("tiny_ragged", dict(), False),                          # no top-K: every page
])
def test_gather_probe_reads_the_attended_tiles(name, ov, null_pages):
    require_gpu()
    say(f"[case] gather probe {name} {ov} null_pages={null_pages}")
    wl = make_workload(name, **ov)
    c = wl.cfg
    ds = DecodeStep(wl, device="cuda")
    cache = ds.caches[0]
    if null_pages:
        pt = cache.page_table.clone()
        pt[:, :, 1::7] = -1
        cache.page_table.copy_(pt)
    q = wl.q(0, device="cuda")
    sel = cnt = None
    if c.topk:
        ds.select(0, q)
        sel, cnt = ds.bufs[0].sel, ds.bufs[0].sel_count
    sink = torch.zeros(kvs.kvs_gather_probe_sink_words(c.d) + 7, dtype=torch.int32, device="cuda")
    kvs.kvs_gather_probe(cache, sel, cnt, c.topk or 0, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy())
    want = _want(cache, None if sel is None else sel.cpu().numpy(),
                 None if cnt is None else cnt.cpu().numpy(), c.P)
    assert got == want
    assert np.all(sink[-7:].cpu().numpy() == 0)                # words past the grid untouched


@pytest.mark.parametrize("nbytes", [16, 16 * 1000, 16 * 64 * 8 * 2 + 48, 48 << 20])
def test_stream_probe_reads_exactly_the_range(nbytes):
    """The plain-read probe folds every word of the first nbytes and nothing
    past them: the XOR over its sink equals the XOR of those words, and a
    poisoned tail beyond nbytes leaves it unchanged."""
    require_gpu()
    say(f"[case] stream probe {nbytes} bytes")
    g = torch.Generator(device="cpu").manual_seed(3)
    words = torch.randint(-2**31, 2**31 - 1, (nbytes // 4 + 1024,), generator=g, dtype=torch.int32)
    src = words.to("cuda")
    sink = torch.zeros(kvs.kvs_stream_probe_sink_words(), dtype=torch.int32, device="cuda")
    kvs.kvs_stream_probe(src, nbytes, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words[: nbytes // 4].numpy().view(np.uint32))
    assert got == want
    with pytest.raises(kvs.KvsError):
        kvs.kvs_stream_probe(src, nbytes + 8, sink)        # not a multiple of 16
    with pytest.raises(kvs.KvsError):
        kvs.kvs_stream_probe(src, nbytes, sink[:1])        # sink too small
