"""KV-cache codec after CacheGen ("CacheGen -- KV Cache Compression and
Streaming", paper notes, sections 3 and 7): one chunk of every layer's K and
V, anchors every ``group`` tokens kept at 8 bits, the other tokens as deltas
to their anchor with a bin per third of the layers, arithmetic coded with
statistics per (channel, layer).  Encoding runs on the host
(``kvs_codec_encode``, offline in the notes), decoding on the GPU
(``kvs_codec_decode``).

Synthetic chunks stand in for a model's KV cache.  The notes' encoder rests
on two properties of real KV data -- neighbouring tokens are close, and each
(channel, layer) has its own range -- so the generator gives every
(layer, K/V, channel) its own scale and offset and lets each channel follow
a first-order autoregressive walk over the tokens.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict

import numpy as np
import torch

from . import kvs

__all__ = ["ChunkConfig", "CHUNKS", "make_chunk"]


@dataclass(frozen=True)
class ChunkConfig:
    name: str
    L: int            # layers
    T: int            # tokens in the chunk
    C: int            # channels per token (all KV heads x head_dim)
    rho: float = 0.9  # token-to-token correlation of each channel
    S: int = 512      # channels per stream
    group: int = 10
    seed: int = 0


CHUNKS: Dict[str, ChunkConfig] = {
    # Llama-7B shapes (32 layers, 32 KV heads x 128) and the notes' default
    # chunk of 1.5K tokens
    "llama7b_chunk": ChunkConfig("llama7b_chunk", L=32, T=1536, C=4096),
    "small_chunk": ChunkConfig("small_chunk", L=6, T=173, C=256, S=128),
}


def make_chunk(cfg: ChunkConfig, device="cpu") -> torch.Tensor:
    """x[L][2][T][C] fp16: per (layer, K/V, channel) a scale
    sigma = exp(N(0, 0.5^2)) and an offset mu = 0.5 sigma N(0, 1); over the
    tokens z_0 ~ N(0, 1), z_t = rho z_{t-1} + sqrt(1 - rho^2) N(0, 1);
    x = mu + sigma z, rounded to fp16."""
    g = torch.Generator(device=device).manual_seed(cfg.seed * 7919 + 17)
    shape = (cfg.L, 2, cfg.C)
    sigma = torch.exp(0.5 * torch.randn(shape, generator=g, device=device))
    mu = 0.5 * sigma * torch.randn(shape, generator=g, device=device)
    x = torch.empty((cfg.L, 2, cfg.T, cfg.C), dtype=torch.float16, device=device)
    z = torch.randn(shape, generator=g, device=device)
    c = float(np.sqrt(1.0 - cfg.rho ** 2))
    for t in range(cfg.T):
        if t:
            z = cfg.rho * z + c * torch.randn(shape, generator=g, device=device)
        x[:, :, t, :] = (mu + sigma * z).to(torch.float16)
    return x


def layout_of(cfg: ChunkConfig) -> kvs.CodecLayout:
    return kvs.codec_layout(cfg.L, cfg.T, cfg.C, cfg.group, cfg.S)


_FIELDS = ("lo", "scale", "tab_first", "tab_n", "tab_off", "cdf", "streams", "stream_off")


def pin(enc: kvs.Encoded) -> kvs.Encoded:
    """The chunk's tensors in pinned host memory (so host-to-device copies run
    asynchronously at the link's rate)."""
    return kvs.Encoded(enc.layout, *[getattr(enc, f).pin_memory() for f in _FIELDS])


class PipelinedLoader:
    """Loads encoded chunks from pinned host memory and decodes them on the
    GPU, the transfer of chunk i overlapping the decode of chunk i - 1
    (CacheGen notes, 7).  Two device buffer sets alternate: the copy of chunk
    i waits for the decode that last read its set, and the decode of chunk i
    waits for its copy.  Both streams keep the default priority."""

    def __init__(self, layout: kvs.CodecLayout, cdf_cap: int, streams_cap: int, device="cuda"):
        L, T, C, S = layout.L, layout.T, layout.C, layout.S
        nstreams = L * 2 * (C // S) * T
        self.layout, self.device = layout, device
        shapes = {"lo": ((L, 2, C), torch.float32), "scale": ((L, 2, C), torch.float32),
                  "tab_first": ((L, 2, C, 2), torch.int32), "tab_n": ((L, 2, C, 2), torch.int32),
                  "tab_off": ((L, 2, C, 2), torch.int32), "cdf": ((cdf_cap,), torch.int16),
                  "streams": ((streams_cap,), torch.uint8),
                  "stream_off": ((nstreams + 1,), torch.int64)}
        self.sets = [{f: torch.empty(s, dtype=dt, device=device) for f, (s, dt) in shapes.items()}
                     for _ in range(2)]
        self.copy_stream = torch.cuda.Stream(device)

    def run(self, chunks, outs) -> None:
        """Decode chunks[i] (pinned host Encoded) into outs[i], in order, on
        the current stream; returns once everything is queued."""
        comp = torch.cuda.current_stream(self.device)
        last_read = [None, None]
        for i, enc in enumerate(chunks):
            k = i % 2
            buf = self.sets[k]
            if enc.cdf.numel() > buf["cdf"].numel() or enc.streams.numel() > buf["streams"].numel():
                raise ValueError("chunk larger than the loader's buffers")
            with torch.cuda.stream(self.copy_stream):
                if last_read[k] is not None:
                    self.copy_stream.wait_event(last_read[k])
                dev = {}
                for f in _FIELDS:
                    src = getattr(enc, f)
                    dst = buf[f] if f not in ("cdf", "streams") else buf[f][:src.numel()]
                    dst.copy_(src, non_blocking=True)
                    dev[f] = dst
                copied = torch.cuda.Event()
                copied.record(self.copy_stream)
            comp.wait_event(copied)
            kvs.kvs_codec_decode(kvs.Encoded(enc.layout, **dev), outs[i], comp)
            done = torch.cuda.Event()
            done.record(comp)
            last_read[k] = done
