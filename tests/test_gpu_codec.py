"""GPU parity of the KV-cache codec decoder (CacheGen notes, sections 3 and
7) through the C ABI: decoded values equal the oracle's quantize-and-
reconstruct bit for bit -- the range coder is lossless and reconstruction is
float32 product-then-sum rounded once to fp16 on both sides -- for streams
written by the library's host encoder and for streams written by the
oracle's own encoder."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_harness import require_gpu, say
from non_uniform_sparse_amd import codec, kvs

pytestmark = pytest.mark.gpu


def _decode(enc: kvs.Encoded) -> np.ndarray:
    lay = enc.layout
    d = enc.to("cuda")
    out = torch.full((lay.L, 2, lay.T, lay.C), float("nan"), dtype=torch.float16, device="cuda")
    kvs.kvs_codec_decode(d, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _want(x: np.ndarray, group: int, bins=(0.5, 1.0, 1.5)) -> np.ndarray:
    lo, scale, sym = O.codec_quantize(x, group, bins)
    return O.codec_reconstruct(lo, scale, sym, group, bins)


@pytest.mark.parametrize("L,T,C,group,S,rho", [
    (3, 23, 16, 10, 8, 0.9),
    (6, 173, 256, 10, 128, 0.9),
    (4, 700, 512, 10, 512, 0.9),     # two workgroups of 640 tokens, the second ragged
    (2, 50, 40, 10, 40, 0.0),        # a block of 32 channels and one of 8
    (3, 100, 64, 16, 32, 0.9),       # 1024 threads per workgroup
    (2, 900, 64, 33, 64, 0.9),       # 31 groups of 33 per workgroup
    (2, 400, 16, 320, 16, 0.5),      # 3 groups of 320
    (3, 12, 16, 1, 16, 0.9),         # anchors only
    (1, 1, 8, 10, 8, 0.5),           # one token
])
def test_decode_matches_oracle(L, T, C, group, S, rho):
    require_gpu()
    say(f"[case] codec L={L} T={T} C={C} group={group} S={S} rho={rho}")
    cfg = codec.ChunkConfig("t", L=L, T=T, C=C, S=S, group=group, rho=rho, seed=T + C)
    x = codec.make_chunk(cfg)
    enc = kvs.kvs_codec_encode(codec.layout_of(cfg), x)
    got = _decode(enc)
    want = _want(x.numpy(), group)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_decode_edge_values():
    require_gpu()
    say("[case] codec edge values")
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1, size=(3, 2, 30, 16)).astype(np.float16)
    x[0, 0, :, 3] = 1.5
    x[1, 1, 5, 7] = 6e4
    x[2, 0, ::10, 2] = np.float16(-0.0)
    for bins in ((0.5, 1.0, 1.5), (0.25, 2.0, 3.0)):
        lay = kvs.codec_layout(3, 30, 16, 10, 8, bins)
        got = _decode(kvs.kvs_codec_encode(lay, torch.from_numpy(x)))
        assert np.array_equal(got.view(np.uint16), _want(x, 10, bins).view(np.uint16))


def test_decode_oracle_written_streams():
    """The GPU decodes bytes the oracle's encoder wrote (tables and streams
    laid out as the C ABI states) to the oracle's own decoded values."""
    require_gpu()
    say("[case] codec oracle streams")
    cfg = codec.ChunkConfig("t", L=3, T=25, C=16, S=8, rho=0.8, seed=3)
    x = codec.make_chunk(cfg).numpy()
    ora = O.codec_encode(x, group=10, S=8)
    L, T, C = 3, 25, 16
    first = np.zeros((L, 2, C, 2), dtype=np.int32)
    n = np.zeros_like(first)
    off = np.zeros_like(first)
    cdf = []
    for l in range(L):
        for kv in range(2):
            for c in range(C):
                for k in range(2):
                    f0, f = ora["tables"][(l, kv, c, k)]
                    first[l, kv, c, k], n[l, kv, c, k], off[l, kv, c, k] = f0, len(f), len(cdf)
                    cdf += np.cumsum([0] + f[:-1]).tolist()
    enc = kvs.Encoded(codec.layout_of(cfg), torch.from_numpy(ora["lo"]),
                      torch.from_numpy(ora["scale"]), torch.from_numpy(first),
                      torch.from_numpy(n), torch.from_numpy(off),
                      torch.from_numpy(np.array(cdf, dtype=np.uint16).view(np.int16)),
                      torch.frombuffer(bytearray(ora["streams"]), dtype=torch.uint8),
                      torch.tensor(ora["offsets"], dtype=torch.int64))
    got = _decode(enc)
    assert np.array_equal(got.view(np.uint16), O.codec_decode(ora).view(np.uint16))


def test_decode_full_size_and_deterministic():
    """The Llama-7B-shaped chunk (32 layers, 4096 channels, 1536 tokens) at the
    stream width the bench uses: every value equals the oracle's; a second
    decode is identical."""
    require_gpu()
    cfg = codec.CHUNKS["llama7b_chunk"]
    say(f"[case] codec full size {cfg}")
    x = codec.make_chunk(cfg)
    enc = kvs.kvs_codec_encode(codec.layout_of(cfg), x)
    d = enc.to("cuda")
    out = torch.empty((cfg.L, 2, cfg.T, cfg.C), dtype=torch.float16, device="cuda")
    kvs.kvs_codec_decode(d, out)
    torch.cuda.synchronize()
    first = out.clone()
    kvs.kvs_codec_decode(d, out)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), out.view(torch.int16))
    got = out.cpu().numpy()
    want = _want(x.numpy(), cfg.group)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    say(f"codec full size: {x.numel() * 2 / 2**20:.0f} MiB fp16 -> {enc.nbytes() / 2**20:.1f} MiB "
        f"({x.numel() * 2 / enc.nbytes():.2f}x)")


def test_pipelined_loader_matches_separate_decodes():
    """Chunks copied and decoded through the two-stream pipeline (transfer of
    chunk i overlapping the decode of chunk i - 1) decode to exactly what
    each chunk decodes to on its own -- more chunks than buffer sets, so the
    sets are reused."""
    require_gpu()
    say("[case] codec pipelined loader")
    cfgs = [codec.ChunkConfig("t", L=3, T=107, C=64, S=32, seed=i) for i in range(4)]
    encs = [kvs.kvs_codec_encode(codec.layout_of(c), codec.make_chunk(c)) for c in cfgs]
    want = [_decode(e) for e in encs]
    cdf_cap = max(e.cdf.numel() for e in encs)
    st_cap = max(e.streams.numel() for e in encs)
    loader = codec.PipelinedLoader(codec.layout_of(cfgs[0]), cdf_cap, st_cap)
    outs = [torch.full((3, 2, 107, 64), float("nan"), dtype=torch.float16, device="cuda")
            for _ in encs]
    loader.run([codec.pin(e) for e in encs], outs)
    torch.cuda.synchronize()
    for o, w in zip(outs, want):
        assert np.array_equal(o.cpu().numpy().view(np.uint16), w.view(np.uint16))
