"""Pins of the codec oracle (CacheGen notes, sections 3 and 7) against
hand-derived bytes, closed forms and invariants -- CPU only."""

import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


@pytest.mark.parametrize("key", ["range_pending_ff", "range_carry"])
def test_range_coder_hand_bytes(key):
    e = GOLDEN[key]
    tabs = [(0, e["freqs"])] * len(e["message"])
    assert O.range_encode(e["message"], tabs).hex() == e["bytes"]
    assert O.range_decode(bytes.fromhex(e["bytes"]), tabs) == e["message"]


def test_table_normalisation_hand_cases():
    for c in GOLDEN["codec_table"]["cases"]:
        assert O.codec_table(c["symbols"]) == (c["first"], c["freqs"])


def test_table_invariants():
    rng = np.random.default_rng(1)
    for _ in range(300):
        n = int(rng.integers(1, 5000))
        syms = rng.integers(-127, 128, size=n) if rng.random() < 0.3 else \
            np.rint(rng.normal(0, rng.uniform(0.2, 20), size=n)).clip(-127, 127).astype(int)
        first, f = O.codec_table(syms)
        assert sum(f) == O.TOTAL and first == syms.min() and first + len(f) - 1 == syms.max()
        present = set(syms.tolist())
        for i, v in enumerate(f):
            assert (v >= 1) == ((first + i) in present)
        cnt = np.bincount(syms - first, minlength=len(f))
        exact = cnt * O.TOTAL / n           # within 1 of the proportional share, except the
        dev = np.abs(np.array(f) - exact)   # symbol that absorbs the rounding
        assert np.sort(dev)[:-1].max(initial=0) <= 1.0
    assert O.codec_table([]) == (0, [O.TOTAL])
    assert O.codec_table([4] * 7) == (4, [O.TOTAL])


def test_range_coder_lossless_and_near_entropy():
    """Round trip over random tables and messages, and the length against
    the ideal code length sum(-log2 p): at most 0.006 bit per symbol lost to
    the truncated r (r = floor(range / 2^16) >= 2^8) plus 6 flush bytes,
    never meaningfully below it."""
    rng = np.random.default_rng(2)
    for _ in range(300):
        n = int(rng.integers(1, 300))
        k = int(rng.integers(1, 40))
        p = rng.dirichlet(np.full(k, rng.uniform(0.1, 2)))
        syms = rng.choice(k, size=n, p=p) - int(rng.integers(-5, 5))
        tab = O.codec_table(syms)
        tabs = [tab] * n
        data = O.range_encode(syms, tabs)
        assert O.range_decode(data, tabs) == syms.tolist()
        ideal = sum(-math.log2(tab[1][s - tab[0]] / O.TOTAL) for s in syms)
        assert ideal - 16 <= 8 * len(data) <= ideal + 0.006 * n + 48


def test_range_coder_mixed_tables_per_symbol():
    """Every symbol with its own table (as channels do): still lossless."""
    rng = np.random.default_rng(3)
    for _ in range(100):
        n = int(rng.integers(1, 200))
        tabs, syms = [], []
        for _ in range(n):
            k = int(rng.integers(1, 9))
            f = O.codec_table(rng.integers(0, k, size=int(rng.integers(1, 50))))
            tabs.append(f)
            nz = [f[0] + i for i, v in enumerate(f[1]) if v]
            syms.append(int(rng.choice(nz)))
        assert O.range_decode(O.range_encode(syms, tabs), tabs) == syms


def test_certain_symbol_costs_nothing():
    """A table with one symbol carries no information: the stream is the
    five flush bytes whatever its length."""
    tab = (0, [O.TOTAL])
    for n in (1, 10, 1000):
        assert O.range_encode([0] * n, [tab] * n) == bytes(5)


def test_layer_bins():
    assert [O.codec_layer_bin(l, 3) for l in range(3)] == [0.5, 1.0, 1.5]
    b = [O.codec_layer_bin(l, 32) for l in range(32)]
    assert (b.count(0.5), b.count(1.0), b.count(1.5)) == (11, 11, 10)
    assert b == sorted(b)


def _chunk(rng, L=3, T=23, C=8, scale=1.0):
    return (rng.normal(0, scale, size=(L, 2, T, C))).astype(np.float16)


def test_quantize_error_bounds_and_ranges():
    rng = np.random.default_rng(4)
    x = _chunk(rng, L=4, T=37, C=16, scale=0.7)
    lo, scale, sym = O.codec_quantize(x)
    xr = O.codec_reconstruct(lo, scale, sym)
    is_anchor = np.arange(37) % 10 == 0
    xf = x.astype(np.float64)
    err = np.abs(xr.astype(np.float64) - xf)
    tol16 = np.abs(xf) * 2.0 ** -10 + 2.0 ** -24
    a_err = err[:, :, is_anchor, :]
    assert np.all(a_err <= scale[:, :, None, :] / 2 * (1 + 1e-6) + tol16[:, :, is_anchor, :] + 1e-7)
    assert sym[:, :, is_anchor, :].min() >= 0 and sym[:, :, is_anchor, :].max() <= 255
    # each anchor range's ends code to 0 and 255
    assert np.all(sym[:, :, is_anchor, :].min(axis=2) == 0)
    assert np.all(sym[:, :, is_anchor, :].max(axis=2) == 255)
    for l in range(4):
        b = O.codec_layer_bin(l, 4)
        d_err = err[l][:, ~is_anchor, :]
        bound = scale[l][:, None, :] / 2 + b / 2
        assert np.all(d_err <= bound * (1 + 1e-6) + tol16[l][:, ~is_anchor, :] + 1e-6)
        assert np.abs(sym[l][:, ~is_anchor, :]).max() <= 127


def test_quantize_hand_values():
    """Two groups, anchors -1 and 1 (codes 0 and 255), deltas at bin 1.0
    (middle layer of three): 0.3 - 1 = -0.7 -> -1 -> 0.0; -1 + 0.6 -> 1 -> 0.0;
    a delta of 300 clamps to 127."""
    x = np.zeros((3, 2, 20, 1), dtype=np.float16)
    x[1, 0, 0, 0], x[1, 0, 10, 0] = -1.0, 1.0
    x[1, 0, 11, 0] = 0.3
    x[1, 0, 1, 0] = -0.4
    x[1, 1, 0, 0], x[1, 1, 10, 0] = 0.0, 0.0
    x[1, 1, 5, 0] = 300.0
    lo, scale, sym = O.codec_quantize(x)
    assert sym[1, 0, 0, 0] == 0 and sym[1, 0, 10, 0] == 255
    assert sym[1, 0, 11, 0] == -1 and sym[1, 0, 1, 0] == 1
    assert scale[1, 1, 0] == 0 and sym[1, 1, 0, 0] == 0 and sym[1, 1, 5, 0] == 127
    xr = O.codec_reconstruct(lo, scale, sym)
    assert xr[1, 0, 11, 0] == np.float16(0.0) and xr[1, 0, 1, 0] == np.float16(0.0)
    assert xr[1, 0, 0, 0] == np.float16(-1.0) and xr[1, 0, 10, 0] == np.float16(1.0)
    assert xr[1, 1, 5, 0] == np.float16(127.0)
    # the same delta of 0.6 in the first (bin 0.5) and last (bin 1.5) layer
    for l, q, val in ((0, 1, -0.5), (2, 0, -1.0)):
        y = np.zeros((3, 2, 20, 1), dtype=np.float16)
        y[l, 0, 0, 0], y[l, 0, 10, 0], y[l, 0, 1, 0] = -1.0, 1.0, -0.4
        lo, scale, sym = O.codec_quantize(y)
        assert sym[l, 0, 1, 0] == q
        assert O.codec_reconstruct(lo, scale, sym)[l, 0, 1, 0] == np.float16(val)


def test_constant_channel_is_exact():
    x = np.full((2, 2, 15, 3), 0.25, dtype=np.float16)
    lo, scale, sym = O.codec_quantize(x)
    assert np.all(scale == 0) and np.all(sym == 0)
    assert np.array_equal(O.codec_reconstruct(lo, scale, sym), x)


def test_chunk_encode_decode_round_trip():
    """Streams decode to exactly the quantized values; stream layout."""
    rng = np.random.default_rng(5)
    x = _chunk(rng, L=3, T=23, C=8)
    for S in (8, 4, 2):
        enc = O.codec_encode(x, S=S)
        assert len(enc["offsets"]) == 3 * 2 * (8 // S) * 23 + 1
        assert all(o % 4 == 0 for o in enc["offsets"])
        lo, scale, sym = O.codec_quantize(x)
        assert np.array_equal(O.codec_decode(enc), O.codec_reconstruct(lo, scale, sym))
