"""The library's host encoder (kvs_codec_encode) against the codec oracle,
byte for byte, and the codec calls' validation -- CPU only (the encoder is
host code)."""

import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from non_uniform_sparse_amd import codec, kvs


def _lib():
    try:
        return kvs.lib()
    except RuntimeError as e:
        pytest.skip(str(e))


def _check_against_oracle(x: np.ndarray, group: int, S: int, bins=(0.5, 1.0, 1.5)):
    L, _, T, C = x.shape
    lay = kvs.codec_layout(L, T, C, group, S, bins)
    e = kvs.kvs_codec_encode(lay, torch.from_numpy(x))
    ora = O.codec_encode(x, group=group, S=S, bins=bins)
    assert np.array_equal(e.lo.numpy(), ora["lo"]) and np.array_equal(e.scale.numpy(), ora["scale"])
    assert e.streams.numpy().tobytes() == ora["streams"]
    assert e.stream_off.tolist() == ora["offsets"]
    cdf = e.cdf.numpy().view(np.uint16)
    first, n, off = (e.tab_first.view(-1).numpy(), e.tab_n.view(-1).numpy(),
                     e.tab_off.view(-1).numpy().view(np.uint32))
    end = 0
    for (l, kv, c, k), (f0, f) in ora["tables"].items():
        i = ((l * 2 + kv) * C + c) * 2 + k
        assert first[i] == f0 and n[i] == len(f) and off[i] == end      # back to back, in order
        assert np.array_equal(cdf[off[i]:off[i] + n[i]], np.cumsum([0] + f[:-1]))
        end += len(f)
    assert end == cdf.size
    return e


@pytest.mark.parametrize("L,T,C,group,S,rho", [
    (3, 23, 16, 10, 8, 0.9),      # ragged last group, two slices
    (4, 40, 32, 10, 32, 0.0),     # iid tokens (wide deltas), one slice
    (2, 7, 8, 10, 8, 0.9),        # a single (partial) group
    (3, 12, 16, 1, 16, 0.9),      # every token an anchor: empty delta tables
    (5, 31, 24, 7, 8, 0.95),      # group 7, L not a multiple of 3
    (1, 1, 8, 10, 8, 0.5),        # one token
])
def test_encoder_matches_oracle(L, T, C, group, S, rho):
    _lib()
    cfg = codec.ChunkConfig("t", L=L, T=T, C=C, S=S, group=group, rho=rho, seed=L * 100 + T)
    _check_against_oracle(codec.make_chunk(cfg).numpy(), group, S)


def test_encoder_edge_values():
    """Constant channels, huge deltas (clamped), signed zeros, custom bins."""
    _lib()
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1, size=(3, 2, 30, 16)).astype(np.float16)
    x[0, 0, :, 3] = 1.5                             # constant channel
    x[1, 1, 5, 7] = 6e4                             # delta clamps at 127
    x[2, 0, ::10, 2] = np.float16(-0.0)
    x[2, 0, 1::10, 2] = np.float16(0.0)
    _check_against_oracle(x, 10, 8)
    _check_against_oracle(x, 10, 16, bins=(0.25, 2.0, 3.0))


def test_codec_validation():
    L = _lib()
    b0, b1 = ctypes.c_uint64(), ctypes.c_uint64()
    ok = dict(L=2, T=10, C=16, group=10, S=8, bins=(0.5, 1.0, 1.5))
    for bad, code in [(dict(S=12), kvs.KVS_EINVAL), (dict(S=32), kvs.KVS_EINVAL),
                      (dict(C=4, S=8), kvs.KVS_EINVAL), (dict(group=0), kvs.KVS_EINVAL),
                      (dict(group=400), kvs.KVS_EINVAL), (dict(T=0), kvs.KVS_EINVAL),
                      (dict(bins=(0.5, 0.0, 1.5)), kvs.KVS_EINVAL),
                      (dict(bins=(0.5, float("inf"), 1.5)), kvs.KVS_EINVAL)]:
        f = {**ok, **bad}
        lay = kvs.codec_layout(f["L"], f["T"], f["C"], f["group"], f["S"], f["bins"])
        assert L.kvs_codec_bounds(ctypes.byref(lay), ctypes.byref(b0), ctypes.byref(b1)) == code
        ch = kvs.CodecChunk(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 10, 0x7000, 0x8000, 64)
        assert L.kvs_codec_decode(ctypes.byref(lay), ctypes.byref(ch), 0x9000, None) == code
    lay = kvs.codec_layout(**{k: v for k, v in ok.items()})
    cdf_max, st_max = kvs.kvs_codec_bounds(lay)
    assert cdf_max == 2 * 2 * 16 * 511 and st_max == 2 * 2 * 2 * 10 * (2 * 8 + 0 + 12)
    ch = kvs.CodecChunk(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 10, 0x7000, 0x8000, 64)
    assert L.kvs_codec_decode(ctypes.byref(lay), ctypes.byref(ch), 0x9008, None) == kvs.KVS_EINVAL
    ch2 = kvs.CodecChunk(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 10, 0x7002, 0x8000, 64)
    assert L.kvs_codec_decode(ctypes.byref(lay), ctypes.byref(ch2), 0x9000, None) == kvs.KVS_EINVAL
    ch3 = kvs.CodecChunk(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0, 10, 0x7000, 0x8000, 64)
    assert L.kvs_codec_decode(ctypes.byref(lay), ctypes.byref(ch3), 0x9000, None) == kvs.KVS_EINVAL


def test_encoder_reports_space_needed():
    L = _lib()
    cfg = codec.ChunkConfig("t", L=2, T=20, C=16, S=8)
    x = codec.make_chunk(cfg)
    lay = codec.layout_of(cfg)
    full = kvs.kvs_codec_encode(lay, x)
    bufs = [torch.empty((2, 2, 16), dtype=torch.float32) for _ in range(2)] + \
        [torch.empty((2, 2, 16, 2), dtype=torch.int32) for _ in range(3)]
    cdf = torch.empty(10, dtype=torch.int16)
    st = torch.empty(16, dtype=torch.uint8)
    off = torch.empty(2 * 2 * 2 * 20 + 1, dtype=torch.int64)
    ch = kvs.CodecChunk(*[b.data_ptr() for b in bufs], cdf.data_ptr(), 10, st.data_ptr(),
                        off.data_ptr(), 16)
    assert L.kvs_codec_encode(ctypes.byref(lay), x.data_ptr(), ctypes.byref(ch), 1) == kvs.KVS_ENOSPC
    assert ch.cdf_len == full.cdf.numel() and ch.streams_len == full.streams.numel()
