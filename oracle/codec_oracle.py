"""Reference KV-cache codec after CacheGen (test infrastructure only).

Follows "CacheGen -- KV Cache Compression and Streaming" (paper notes),
section 3 (change-based encoding over groups of tokens) and section 7
(implementation details: anchors kept at 8 bits, deltas quantized with a
bin per third of the layers, arithmetic coding with statistics per channel
and layer, one GPU thread decoding each token's symbols).  Where the notes
leave a step open the plainest reading is taken:

  * one chunk is x[L][2][T][C]: layer, K (0) / V (1), token, channel (all KV
    heads' channels of the token side by side), fp16;
  * token t is the anchor of its group iff t % group == 0; the others are
    stored as the delta to their group's anchor (the original anchor value:
    an error in the anchor carries into the whole group, the reason the
    notes give for keeping anchors at 8 bits);
  * layer l belongs to third floor(3 l / L), whose delta bin is
    bins[floor(3 l / L)];
  * the 8-bit anchor code is uniform over [min, max] of the chunk's anchors
    of that (layer, K/V, channel), 255 steps; a constant channel codes 0;
  * a delta symbol is round-half-even(delta / bin), clamped to [-127, 127];
  * every (layer, K/V, channel) has two symbol tables -- anchors and deltas
    -- built from the chunk's own symbol counts, normalized to a total of
    2^16 with every present symbol at least 1;
  * the entropy coder is a 32-bit byte-wise range coder (an integer form
    of arithmetic coding) with carry propagation through pending 0xFF
    bytes;
  * a stream holds the symbols of one token over S consecutive channels,
    in channel order; streams are padded to 4 bytes.

All arithmetic that decides an integer (a quantized code) is done in IEEE
float32, as written; reconstruction is float32 (product, then sum) rounded
to fp16.  The range coder is pure Python integers: use it on small inputs.
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

__all__ = [
    "codec_layer_bin",
    "codec_quantize",
    "codec_reconstruct",
    "codec_table",
    "range_encode",
    "range_decode",
    "codec_encode",
    "codec_decode",
    "TOTAL",
]

TOTAL = 1 << 16          # frequency total of every table
_TOP = 1 << 24           # renormalize while the range is below this


# ------------------------------------------------------------ quantization --

def codec_layer_bin(l: int, L: int, bins: Sequence[float] = (0.5, 1.0, 1.5)) -> float:
    """Delta bin of layer l: the layers are cut into three equal groups,
    shallow to deep (CacheGen notes, section 7, default quantization)."""
    return float(bins[(3 * l) // L])


def codec_quantize(x: np.ndarray, group: int = 10, bins: Sequence[float] = (0.5, 1.0, 1.5)):
    """x: [L][2][T][C] float16.  Returns (lo, scale, sym): lo and scale
    [L][2][C] float32 of the anchor code, sym [L][2][T][C] int32 holding the
    anchor code (0..255) at anchor tokens and the delta symbol (-127..127)
    elsewhere."""
    x = np.asarray(x, dtype=np.float16).astype(np.float32)
    L, two, T, C = x.shape
    is_anchor = (np.arange(T) % group) == 0
    anchors = x[:, :, is_anchor, :]                                  # [L][2][A][C]
    lo = anchors.min(axis=2)
    hi = anchors.max(axis=2)
    scale = ((hi - lo) / np.float32(255.0)).astype(np.float32)
    sym = np.zeros(x.shape, dtype=np.int32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = np.rint((anchors - lo[:, :, None, :]) / safe[:, :, None, :])
    codes = np.where(scale[:, :, None, :] > 0, np.clip(codes, 0, 255), 0)
    sym[:, :, is_anchor, :] = codes.astype(np.int32)
    anchor_of = (np.arange(T) // group) * group
    for l in range(L):
        b = np.float32(codec_layer_bin(l, L, bins))
        d = (x[l] - x[l][:, anchor_of, :]) / b                          # [2][T][C] float32
        q = np.clip(np.rint(d), -127, 127).astype(np.int32)
        sym[l][:, ~is_anchor, :] = q[:, ~is_anchor, :]
    return lo.astype(np.float32), scale, sym


def codec_reconstruct(lo: np.ndarray, scale: np.ndarray, sym: np.ndarray, group: int = 10,
                      bins: Sequence[float] = (0.5, 1.0, 1.5)) -> np.ndarray:
    """Decoded values [L][2][T][C] float16: an anchor is lo + code*scale, a
    delta token its anchor's decoded value + q*bin (float32, product then
    sum, rounded once to fp16)."""
    L, two, T, C = sym.shape
    is_anchor = (np.arange(T) % group) == 0
    anchor_of = (np.arange(T) // group) * group
    a = (lo[:, :, None, :] + sym.astype(np.float32) * scale[:, :, None, :]).astype(np.float32)
    out = np.empty(sym.shape, dtype=np.float32)
    for l in range(L):
        b = np.float32(codec_layer_bin(l, L, bins))
        base = a[l][:, anchor_of, :]
        out[l] = np.where(is_anchor[None, :, None], a[l],
                          (base + (sym[l].astype(np.float32) * b)).astype(np.float32))
    return out.astype(np.float16)


# ----------------------------------------------------------------- tables --

def codec_table(symbols: Sequence[int]) -> Tuple[int, List[int]]:
    """Frequency table of one (layer, K/V, channel, kind): (first symbol,
    frequencies over [first, last] present symbol).  Each present symbol gets
    floor(count * 2^16 / n), at least 1; absent symbols in between get 0; the
    difference to 2^16 goes to the largest frequency (ties: the lowest
    symbol).  No symbols at all: the single symbol 0 with the whole total."""
    symbols = [int(s) for s in symbols]
    if not symbols:
        return 0, [TOTAL]
    lo, hi = min(symbols), max(symbols)
    counts = [0] * (hi - lo + 1)
    for s in symbols:
        counts[s - lo] += 1
    n = len(symbols)
    f = [max(1, c * TOTAL // n) if c else 0 for c in counts]
    big = max(range(len(f)), key=lambda i: (f[i], -i))
    f[big] += TOTAL - sum(f)
    return lo, f


def _cdf(freqs: Sequence[int]) -> List[int]:
    c = [0]
    for v in freqs:
        c.append(c[-1] + v)
    return c


# ----------------------------------------------------------- range coder --

def range_encode(symbols: Sequence[int], tables: Sequence[Tuple[int, Sequence[int]]]) -> bytes:
    """Encode symbols[i] with table tables[i] = (first symbol, frequencies).

    State: low (33 bits: bit 32 is a carry), range (32 bits), the last byte
    not yet written (`cache`) and the count of bytes held back behind it
    (`pending`, the cache itself plus any 0xFF bytes a later carry would
    turn to 0x00).  Each symbol narrows [low, low + range) to its slice of
    width r*f with r = floor(range / 2^16); while range < 2^24 the top byte
    of low leaves (shift) and range grows by 8 bits.  Five shifts flush."""
    low, rng, cache, pending = 0, 0xFFFFFFFF, 0, 1
    out = bytearray()

    def shift():
        nonlocal low, cache, pending
        if low < 0xFF000000 or low >= (1 << 32):
            carry = low >> 32
            out.append((cache + carry) & 0xFF)
            for _ in range(pending - 1):
                out.append((0xFF + carry) & 0xFF)
            pending = 0
            cache = (low >> 24) & 0xFF
        pending += 1
        low = (low & 0x00FFFFFF) << 8

    for s, (first, freqs) in zip(symbols, tables):
        i = int(s) - first
        if not 0 <= i < len(freqs) or freqs[i] == 0:
            raise ValueError(f"symbol {s} is not in its table")
        cdf = _cdf(freqs)
        r = rng >> 16
        low += r * cdf[i]
        rng = r * freqs[i]
        while rng < _TOP:
            rng <<= 8
            shift()
    for _ in range(5):
        shift()
    return bytes(out)


def range_decode(data: bytes, tables: Sequence[Tuple[int, Sequence[int]]]) -> List[int]:
    """Inverse of range_encode: one symbol per table.  The code register
    holds the stream's bytes aligned with the encoder's low; the symbol is
    the one whose cumulative slice holds floor(code / r).  Bytes past the
    end read as 0."""
    pos = 0

    def byte():
        nonlocal pos
        b = data[pos] if pos < len(data) else 0
        pos += 1
        return b

    code, rng = 0, 0xFFFFFFFF
    for _ in range(5):
        code = ((code << 8) | byte()) & 0xFFFFFFFF
    out = []
    for first, freqs in tables:
        cdf = _cdf(freqs)
        r = rng >> 16
        v = min(code // r, TOTAL - 1)
        i = max(k for k in range(len(freqs)) if cdf[k] <= v and freqs[k] > 0)
        code -= r * cdf[i]
        rng = r * freqs[i]
        while rng < _TOP:
            rng <<= 8
            code = ((code << 8) | byte()) & 0xFFFFFFFF
        out.append(first + i)
    return out


# ------------------------------------------------------------ whole chunk --

def codec_encode(x: np.ndarray, group: int = 10, S: int = 0,
                 bins: Sequence[float] = (0.5, 1.0, 1.5)) -> Dict[str, object]:
    """Encode one chunk.  S: channels per stream (0: all C).  Returns lo,
    scale, tables {(l, kv, c, kind): (first, freqs)} with kind 0 = anchor,
    1 = delta, and the streams in order ((l*2 + kv)*(C/S) + slice)*T + t,
    each padded with zero bytes to a multiple of 4, with byte offsets."""
    lo, scale, sym = codec_quantize(x, group, bins)
    L, two, T, C = sym.shape
    S = S or C
    if C % S:
        raise ValueError("S must divide C")
    is_anchor = (np.arange(T) % group) == 0
    tables = {}
    for l in range(L):
        for kv in range(2):
            for c in range(C):
                tables[(l, kv, c, 0)] = codec_table(sym[l, kv, is_anchor, c])
                tables[(l, kv, c, 1)] = codec_table(sym[l, kv, ~is_anchor, c])
    streams, offsets = bytearray(), [0]
    for l in range(L):
        for kv in range(2):
            for sl in range(C // S):
                for t in range(T):
                    kind = 0 if is_anchor[t] else 1
                    chans = range(sl * S, (sl + 1) * S)
                    b = range_encode([sym[l, kv, t, c] for c in chans],
                                     [tables[(l, kv, c, kind)] for c in chans])
                    b += bytes(-len(b) % 4)
                    streams += b
                    offsets.append(len(streams))
    return {"lo": lo, "scale": scale, "tables": tables, "streams": bytes(streams),
            "offsets": offsets, "shape": (L, T, C), "group": group, "S": S,
            "bins": tuple(bins), "sym": sym}


def codec_decode(enc: Dict[str, object]) -> np.ndarray:
    """Decode a chunk from its streams and tables (the range decoder, then
    the reconstruction)."""
    L, T, C = enc["shape"]
    group, S = enc["group"], enc["S"]
    is_anchor = (np.arange(T) % group) == 0
    sym = np.zeros((L, 2, T, C), dtype=np.int32)
    data, off, tables = enc["streams"], enc["offsets"], enc["tables"]
    s = 0
    for l in range(L):
        for kv in range(2):
            for sl in range(C // S):
                for t in range(T):
                    kind = 0 if is_anchor[t] else 1
                    chans = list(range(sl * S, (sl + 1) * S))
                    sym[l, kv, t, chans] = range_decode(
                        data[off[s]:off[s + 1]], [tables[(l, kv, c, kind)] for c in chans])
                    s += 1
    return codec_reconstruct(enc["lo"], enc["scale"], sym, group, enc["bins"])
