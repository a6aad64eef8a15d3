"""ctypes binding of libkvs.so.  Argument marshalling only: every step of
the decode path runs in the library's HIP kernels or its C++ host code.
Function names match the C entry points declared in include/kvs.h.

Device buffers are torch tensors on a ROCm device; streams are torch
streams (the current stream by default).  A missing library raises at
first use -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvs.so")

KVS_OK, KVS_EINVAL, KVS_EUNSUPPORTED, KVS_EHIP, KVS_ENOSPC = 0, -1, -2, -3, -4
KVS_F16, KVS_BF16 = 0, 1
KVS_PAGE_ON_HOST = -2

# Every symbol include/kvs.h declares.
EXPORTS = (
    "kvs_build_minmax", "kvs_score_pages", "kvs_score_pages_heads", "kvs_topk_pages",
    "kvs_topk_pages_heads", "kvs_select_pages", "kvs_append_kv", "kvs_prefill_chunk",
    "kvs_prefill_workspace_bytes",
    "kvs_offload_pages", "kvs_promote_pages", "kvs_append_kv_tier",
    "kvs_codec_bounds", "kvs_codec_encode", "kvs_codec_decode",
    "kvs_gather_probe", "kvs_gather_probe_sink_words", "kvs_stream_probe",
    "kvs_stream_probe_sink_words",
    "kvs_plan_split", "kvs_prefill_quota", "kvs_rerank_heads",
    "kvs_decode_attn", "kvs_decode_splits", "kvs_decode_combine", "kvs_decode_attn_noalloc",
    "kvs_decode_workspace_bytes", "kvs_decode_concurrency", "kvs_cluster_heads",
    "kvs_last_error",
)


class KvsError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class PagedKV(ctypes.Structure):
    _fields_ = [
        ("kv", ctypes.c_void_p),
        ("minmax", ctypes.c_void_p),
        ("meta_base", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("seq_len", ctypes.c_void_p),
        ("head_slot", ctypes.c_void_p),
        ("b", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Hp", ctypes.c_int32), ("d", ctypes.c_int32), ("P", ctypes.c_int32),
        ("max_group_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("num_meta", ctypes.c_int32), ("dtype", ctypes.c_int32),
    ]


class HostTier(ctypes.Structure):
    _fields_ = [
        ("host_kv", ctypes.c_void_p),
        ("host_base", ctypes.c_void_p),
        ("slot_page", ctypes.c_void_p),
        ("slot_phys", ctypes.c_void_p),
        ("slots", ctypes.c_int32),
        ("num_host_pages", ctypes.c_int64),
    ]


class CodecLayout(ctypes.Structure):
    _fields_ = [
        ("L", ctypes.c_int32), ("T", ctypes.c_int32), ("C", ctypes.c_int32),
        ("group", ctypes.c_int32), ("S", ctypes.c_int32), ("bins", ctypes.c_float * 3),
    ]


class CodecChunk(ctypes.Structure):
    _fields_ = [
        ("lo", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("tab_first", ctypes.c_void_p),
        ("tab_n", ctypes.c_void_p), ("tab_off", ctypes.c_void_p), ("cdf", ctypes.c_void_p),
        ("cdf_len", ctypes.c_uint64), ("streams", ctypes.c_void_p),
        ("stream_off", ctypes.c_void_p), ("streams_len", ctypes.c_uint64),
    ]


_lib = None


def use_library(path: str) -> None:
    """Select which build of the library to load (before its first use), e.g.
    the workgroup-stamp instrumented one for skew measurements."""
    global LIB_PATH
    if _lib is not None:
        raise RuntimeError("library already loaded")
    LIB_PATH = path


def lib() -> ctypes.CDLL:
    """Load libkvs.so (built in-tree by ``python -m non_uniform_sparse_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m non_uniform_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_double
        pkv = ctypes.POINTER(PagedKV)
        L.kvs_build_minmax.argtypes = [pkv, vp]
        L.kvs_score_pages.argtypes = [pkv, vp, vp, vp]
        L.kvs_score_pages_heads.argtypes = [pkv, vp, vp, vp, vp]
        L.kvs_topk_pages.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
        L.kvs_topk_pages_heads.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
        L.kvs_select_pages.argtypes = [pkv, vp, vp, i32, vp, vp, vp]
        L.kvs_append_kv.argtypes = [pkv, vp, vp, vp]
        L.kvs_prefill_chunk.argtypes = [pkv, vp, vp, vp, vp, i32, vp, ctypes.c_size_t, vp]
        L.kvs_prefill_workspace_bytes.argtypes = [i32, i32, i32]
        L.kvs_prefill_workspace_bytes.restype = ctypes.c_size_t
        ptier = ctypes.POINTER(HostTier)
        L.kvs_offload_pages.argtypes = [pkv, ptier, vp]
        L.kvs_promote_pages.argtypes = [pkv, ptier, vp, vp, i32, vp, vp, vp]
        L.kvs_append_kv_tier.argtypes = [pkv, ptier, vp, vp, vp]
        play, pch = ctypes.POINTER(CodecLayout), ctypes.POINTER(CodecChunk)
        L.kvs_codec_bounds.argtypes = [play, ctypes.POINTER(ctypes.c_uint64),
                                       ctypes.POINTER(ctypes.c_uint64)]
        L.kvs_codec_encode.argtypes = [play, vp, pch, i32]
        L.kvs_codec_decode.argtypes = [play, pch, vp, vp]
        L.kvs_gather_probe.argtypes = [pkv, vp, vp, i32, vp, ctypes.c_size_t, vp]
        L.kvs_gather_probe_sink_words.argtypes = [i32, ctypes.POINTER(i32)]
        L.kvs_stream_probe.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp]
        L.kvs_stream_probe_sink_words.argtypes = [ctypes.POINTER(i32)]
        L.kvs_plan_split.argtypes = [vp, vp, i32, i32, i32, f64, i32, vp]
        L.kvs_prefill_quota.argtypes = [vp, vp, i32, i32, ctypes.c_int64, i32, vp]
        L.kvs_rerank_heads.argtypes = [vp, i32, i32, i32, vp]
        for name in ("kvs_decode_attn", "kvs_decode_splits", "kvs_decode_combine"):
            getattr(L, name).argtypes = [pkv, vp, vp, vp, i32, vp, f32, vp, ctypes.c_size_t, vp, vp]
        L.kvs_decode_attn_noalloc.argtypes = [pkv, vp, vp, vp, i32, vp, f32, vp, vp]
        L.kvs_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, vp, i32]
        L.kvs_decode_workspace_bytes.restype = ctypes.c_size_t
        L.kvs_decode_concurrency.argtypes = [i32, i32, i32, i32, vp]
        L.kvs_cluster_heads.argtypes = [vp, i32, i32, i32, vp]
        L.kvs_last_error.restype = ctypes.c_char_p
        if hasattr(L, "kvs_decode_stamps_offset"):   # instrumented build only
            L.kvs_decode_stamps_offset.argtypes = [i32, i32, i32, i32, vp, i32]
            L.kvs_decode_stamps_offset.restype = ctypes.c_size_t
            L.kvs_score_stamps.argtypes = [vp, ctypes.c_size_t, vp]
            L.kvs_score_stamps.restype = ctypes.c_int
            L.kvs_select_stamps.argtypes = [vp, ctypes.c_size_t, vp]
            L.kvs_select_stamps.restype = ctypes.c_int
        for name in EXPORTS:
            if name not in ("kvs_decode_workspace_bytes", "kvs_prefill_workspace_bytes",
                            "kvs_last_error"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def last_error() -> str:
    return lib().kvs_last_error().decode()


def _check(rc: int) -> None:
    if rc != KVS_OK:
        raise KvsError(rc, last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def dtype_code(t: torch.dtype) -> int:
    return {torch.float16: KVS_F16, torch.bfloat16: KVS_BF16}[t]


def _need(t: torch.Tensor, name: str, shape, dtype, device=None) -> None:
    """Shape / dtype / layout check of a tensor handed to the library."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


@dataclass
class Cache:
    """One layer's paged KV as device tensors (the fields of kvs_paged_kv)."""
    kv: torch.Tensor            # [num_pages][Hp][2][P][d]
    minmax: torch.Tensor        # [num_meta][d][2], per-head runs in page order
    meta_base: torch.Tensor     # int32 [b][Hkv]: first min-max block of each head
    page_table: torch.Tensor    # int32 [b][G][max_group_pages]
    seq_len: torch.Tensor       # int32 [b][Hkv]
    head_slot: torch.Tensor     # int32 [Hkv]
    Hq: int

    def rows(self, r0: int, r1: int) -> "Cache":
        """The requests [r0, r1) as a cache of their own: views of the
        per-request tables over the same pool and min-max cache."""
        return Cache(kv=self.kv, minmax=self.minmax, meta_base=self.meta_base[r0:r1],
                     page_table=self.page_table[r0:r1], seq_len=self.seq_len[r0:r1],
                     head_slot=self.head_slot, Hq=self.Hq)

    def struct(self) -> PagedKV:
        num_pages, Hp, two, P, d = self.kv.shape
        b, G, maxpg = self.page_table.shape
        Hkv = self.seq_len.shape[1]
        dev = self.kv.device
        _need(self.kv, "kv", (num_pages, Hp, 2, P, d), self.kv.dtype, dev)
        num_meta = self.minmax.shape[0]
        _need(self.minmax, "minmax", (num_meta, d, 2), self.kv.dtype, dev)
        _need(self.meta_base, "meta_base", (b, Hkv), torch.int32, dev)
        _need(self.page_table, "page_table", (b, Hkv // Hp, maxpg), torch.int32, dev)
        _need(self.seq_len, "seq_len", (b, Hkv), torch.int32, dev)
        _need(self.head_slot, "head_slot", (Hkv,), torch.int32, dev)
        return PagedKV(self.kv.data_ptr(), self.minmax.data_ptr(), self.meta_base.data_ptr(),
                       self.page_table.data_ptr(), self.seq_len.data_ptr(),
                       self.head_slot.data_ptr(), b, self.Hq, Hkv, Hp, d, P, maxpg, num_pages,
                       num_meta, dtype_code(self.kv.dtype))


def kvs_build_minmax(cache: Cache, stream=None) -> None:
    s = cache.struct()
    _check(lib().kvs_build_minmax(ctypes.byref(s), _stream(stream)))


def _heads(heads, Hkv: int) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(heads, dtype=bool).astype(np.uint8))
    if h.shape != (Hkv,):
        raise ValueError(f"heads must have one entry per KV head ({Hkv})")
    return h


def kvs_score_pages(cache: Cache, q: torch.Tensor, scores: torch.Tensor, stream=None,
                    heads=None) -> None:
    """Score every page (heads=None) or only those of the KV heads with
    heads[h] true; the other heads' rows are left as they are."""
    s = cache.struct()
    _need(q, "q", (s.b, s.Hq, s.d), cache.kv.dtype, cache.kv.device)
    _need(scores, "scores", (s.b, s.Hkv, s.max_group_pages), torch.float32, cache.kv.device)
    if heads is None:
        _check(lib().kvs_score_pages(ctypes.byref(s), _ptr(q), _ptr(scores), _stream(stream)))
    else:
        h = _heads(heads, s.Hkv)
        _check(lib().kvs_score_pages_heads(ctypes.byref(s), _ptr(q), h.ctypes.data, _ptr(scores),
                                           _stream(stream)))


def kvs_topk_pages(scores: torch.Tensor, seq_len: torch.Tensor, P: int, K: int,
                   sel: torch.Tensor, sel_count: torch.Tensor, stream=None, heads=None) -> None:
    """Top-K of every head (heads=None) or only of the KV heads with heads[h]
    true; the other heads keep their selection."""
    b, Hkv, max_pages = scores.shape
    _need(scores, "scores", (b, Hkv, max_pages), torch.float32)
    _need(seq_len, "seq_len", (b, Hkv), torch.int32, scores.device)
    _need(sel, "sel", (b, Hkv, K), torch.int32, scores.device)
    _need(sel_count, "sel_count", (b, Hkv), torch.int32, scores.device)
    if heads is None:
        _check(lib().kvs_topk_pages(_ptr(scores), _ptr(seq_len), P, b, Hkv, max_pages, K,
                                    _ptr(sel), _ptr(sel_count), _stream(stream)))
    else:
        h = _heads(heads, Hkv)
        _check(lib().kvs_topk_pages_heads(_ptr(scores), _ptr(seq_len), P, b, Hkv, max_pages, K,
                                          h.ctypes.data, _ptr(sel), _ptr(sel_count),
                                          _stream(stream)))


def kvs_select_pages(cache: Cache, q: torch.Tensor, scores: Optional[torch.Tensor], K: int,
                     sel: torch.Tensor, sel_count: torch.Tensor, stream=None) -> None:
    """Scores and top-K of every head in one launch; scores may be None."""
    s = cache.struct()
    dev = cache.kv.device
    _need(q, "q", (s.b, s.Hq, s.d), cache.kv.dtype, dev)
    if scores is not None:
        _need(scores, "scores", (s.b, s.Hkv, s.max_group_pages), torch.float32, dev)
    _need(sel, "sel", (s.b, s.Hkv, K), torch.int32, dev)
    _need(sel_count, "sel_count", (s.b, s.Hkv), torch.int32, dev)
    _check(lib().kvs_select_pages(ctypes.byref(s), _ptr(q), _ptr(scores), K, _ptr(sel),
                                  _ptr(sel_count), _stream(stream)))


def kvs_append_kv(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    """Append one token per (request, KV head) and update its page's bounds;
    advances the cache's seq_len on the device."""
    s = cache.struct()
    dev = cache.kv.device
    _need(k_new, "k_new", (s.b, s.Hkv, s.d), cache.kv.dtype, dev)
    _need(v_new, "v_new", (s.b, s.Hkv, s.d), cache.kv.dtype, dev)
    _check(lib().kvs_append_kv(ctypes.byref(s), _ptr(k_new), _ptr(v_new), _stream(stream)))


@dataclass
class Tier:
    """Host tier of one layer's cache (the fields of kvs_host_tier)."""
    host_kv: torch.Tensor       # pinned host [num_host_pages][2][P][d]
    host_base: torch.Tensor     # int64 [b][Hkv], -1: head not tiered
    slot_page: torch.Tensor     # int32 [b][Hkv][slots], -1 free
    slot_phys: torch.Tensor     # int32 [b][Hkv][slots]

    def struct(self, cache: Cache) -> HostTier:
        b, Hkv = cache.seq_len.shape
        dev = cache.kv.device
        _, _, two, P, d = cache.kv.shape
        if not self.host_kv.is_pinned():
            raise ValueError("host_kv must be pinned host memory")
        _need(self.host_kv, "host_kv", (self.host_kv.shape[0], 2, P, d), cache.kv.dtype,
              torch.device("cpu"))
        slots = self.slot_page.shape[2]
        _need(self.host_base, "host_base", (b, Hkv), torch.int64, dev)
        _need(self.slot_page, "slot_page", (b, Hkv, slots), torch.int32, dev)
        _need(self.slot_phys, "slot_phys", (b, Hkv, slots), torch.int32, dev)
        return HostTier(self.host_kv.data_ptr(), self.host_base.data_ptr(),
                        self.slot_page.data_ptr(), self.slot_phys.data_ptr(), slots,
                        self.host_kv.shape[0])


def kvs_offload_pages(cache: Cache, tier: Tier, stream=None) -> None:
    """Copy every resident page of the tiered heads to its host page."""
    s, t = cache.struct(), tier.struct(cache)
    _check(lib().kvs_offload_pages(ctypes.byref(s), ctypes.byref(t), _stream(stream)))


def kvs_append_kv_tier(cache: Cache, tier: Tier, k_new: torch.Tensor, v_new: torch.Tensor,
                       stream=None) -> None:
    """kvs_append_kv with the tiered heads' rows written through to their
    host pages."""
    s, t = cache.struct(), tier.struct(cache)
    dev = cache.kv.device
    _need(k_new, "k_new", (s.b, s.Hkv, s.d), cache.kv.dtype, dev)
    _need(v_new, "v_new", (s.b, s.Hkv, s.d), cache.kv.dtype, dev)
    _check(lib().kvs_append_kv_tier(ctypes.byref(s), ctypes.byref(t), _ptr(k_new), _ptr(v_new),
                                    _stream(stream)))


def kvs_promote_pages(cache: Cache, tier: Tier, sel: torch.Tensor, sel_count: torch.Tensor,
                      K: int, heads=None, moved: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """Make the selection of the tiered heads (heads=None: every head)
    resident, moving only the newly selected pages from the host tier."""
    s, t = cache.struct(), tier.struct(cache)
    dev = cache.kv.device
    _need(sel, "sel", (s.b, s.Hkv, K), torch.int32, dev)
    _need(sel_count, "sel_count", (s.b, s.Hkv), torch.int32, dev)
    if moved is not None:
        _need(moved, "moved", (s.b, s.Hkv), torch.int32, dev)
    h = None if heads is None else _heads(heads, s.Hkv)
    _check(lib().kvs_promote_pages(ctypes.byref(s), ctypes.byref(t), _ptr(sel), _ptr(sel_count),
                                   K, None if h is None else h.ctypes.data, _ptr(moved),
                                   _stream(stream)))


@dataclass
class Encoded:
    """One encoded chunk: the fields of kvs_codec_chunk as tensors (host
    after kvs_codec_encode; ``to`` copies them to a device)."""
    layout: CodecLayout
    lo: torch.Tensor           # float32 [L][2][C]
    scale: torch.Tensor        # float32 [L][2][C]
    tab_first: torch.Tensor    # int32 [L][2][C][2]
    tab_n: torch.Tensor        # int32 [L][2][C][2]
    tab_off: torch.Tensor      # int32 holding uint32 [L][2][C][2]
    cdf: torch.Tensor          # int16 holding uint16 [entries]
    streams: torch.Tensor      # uint8 [bytes]
    stream_off: torch.Tensor   # int64 [streams + 1]

    def to(self, device) -> "Encoded":
        f = {k: getattr(self, k).to(device) for k in
             ("lo", "scale", "tab_first", "tab_n", "tab_off", "cdf", "streams", "stream_off")}
        return Encoded(self.layout, **f)

    def struct(self) -> CodecChunk:
        return CodecChunk(self.lo.data_ptr(), self.scale.data_ptr(), self.tab_first.data_ptr(),
                          self.tab_n.data_ptr(), self.tab_off.data_ptr(), self.cdf.data_ptr(),
                          self.cdf.numel(), self.streams.data_ptr(),
                          self.stream_off.data_ptr(), self.streams.numel())

    def nbytes(self) -> int:
        """Bytes of the encoded chunk: streams, offsets, tables, ranges."""
        return sum(t.numel() * t.element_size() for t in
                   (self.lo, self.scale, self.tab_first, self.tab_n, self.tab_off, self.cdf,
                    self.streams, self.stream_off))


def codec_layout(L: int, T: int, C: int, group: int = 10, S: int = 512,
                 bins=(0.5, 1.0, 1.5)) -> CodecLayout:
    return CodecLayout(L, T, C, group, S, (ctypes.c_float * 3)(*bins))


def kvs_codec_bounds(layout: CodecLayout):
    a, b = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().kvs_codec_bounds(ctypes.byref(layout), ctypes.byref(a), ctypes.byref(b)))
    return int(a.value), int(b.value)


def kvs_codec_encode(layout: CodecLayout, x: torch.Tensor, threads: int = 0) -> Encoded:
    """Encode x (host fp16 [L][2][T][C]) on the host."""
    L, T, C, S = layout.L, layout.T, layout.C, layout.S
    _need(x, "x", (L, 2, T, C), torch.float16, torch.device("cpu"))
    cdf_max, _ = kvs_codec_bounds(layout)
    nstreams = L * 2 * (C // S) * T
    guess = x.numel() * 2 // 2 + 64 * nstreams
    while True:
        e = Encoded(layout,
                    torch.empty((L, 2, C), dtype=torch.float32),
                    torch.empty((L, 2, C), dtype=torch.float32),
                    torch.empty((L, 2, C, 2), dtype=torch.int32),
                    torch.empty((L, 2, C, 2), dtype=torch.int32),
                    torch.empty((L, 2, C, 2), dtype=torch.int32),
                    torch.empty(cdf_max, dtype=torch.int16),
                    torch.empty(guess, dtype=torch.uint8),
                    torch.empty(nstreams + 1, dtype=torch.int64))
        s = e.struct()
        rc = lib().kvs_codec_encode(ctypes.byref(layout), _ptr(x), ctypes.byref(s), threads)
        if rc == KVS_ENOSPC and s.streams_len > guess:
            guess = int(s.streams_len)
            continue
        _check(rc)
        e.cdf = e.cdf[:s.cdf_len].clone()
        e.streams = e.streams[:s.streams_len].clone()
        return e


def kvs_codec_decode(enc: Encoded, out: torch.Tensor, stream=None) -> None:
    """Decode a device-resident chunk into out (device fp16 [L][2][T][C])."""
    lay = enc.layout
    _need(out, "out", (lay.L, 2, lay.T, lay.C), torch.float16, enc.streams.device)
    s = enc.struct()
    _check(lib().kvs_codec_decode(ctypes.byref(lay), ctypes.byref(s), _ptr(out), _stream(stream)))


def kvs_gather_probe_sink_words(d: int) -> int:
    w = ctypes.c_int32()
    _check(lib().kvs_gather_probe_sink_words(d, ctypes.byref(w)))
    return int(w.value)


def kvs_gather_probe(cache: Cache, sel: Optional[torch.Tensor], sel_count: Optional[torch.Tensor],
                     K: int, sink: torch.Tensor, stream=None) -> None:
    """Read every attended K/V tile through the page table, no arithmetic
    (the empirical ceiling of the decode's gather)."""
    s = cache.struct()
    dev = cache.kv.device
    if sel is not None:
        _need(sel, "sel", (s.b, s.Hkv, K), torch.int32, dev)
        _need(sel_count, "sel_count", (s.b, s.Hkv), torch.int32, dev)
    if sink.dtype != torch.int32 or not sink.is_contiguous() or sink.device != dev:
        raise ValueError("sink: contiguous int32 on the cache's device")
    _check(lib().kvs_gather_probe(ctypes.byref(s), _ptr(sel), _ptr(sel_count), K, _ptr(sink),
                                  sink.numel(), _stream(stream)))


def kvs_stream_probe_sink_words() -> int:
    w = ctypes.c_int32(0)
    _check(lib().kvs_stream_probe_sink_words(ctypes.byref(w)))
    return w.value


def kvs_stream_probe(src: torch.Tensor, nbytes: int, sink: torch.Tensor, stream=None) -> None:
    """Plain read of the first ``nbytes`` bytes of ``src`` (a contiguous device
    tensor); one XOR word per wave into ``sink`` (int32)."""
    if not src.is_contiguous() or nbytes > src.numel() * src.element_size():
        raise ValueError("src must be contiguous and hold nbytes")
    _check(lib().kvs_stream_probe(_ptr(src), int(nbytes), _ptr(sink), sink.numel(),
                                  _stream(stream)))


def kvs_prefill_workspace_bytes(b: int, Hkv: int, C: int) -> int:
    return int(lib().kvs_prefill_workspace_bytes(b, Hkv, C))


def kvs_prefill_chunk(cache: Cache, k_chunk: torch.Tensor, v_chunk: torch.Tensor,
                      scores: torch.Tensor, quota: torch.Tensor, workspace: torch.Tensor,
                      stream=None) -> None:
    """Keep each head's quota best tokens of a prefill chunk, append them to
    its pages, update their bounds and advance seq_len on the device."""
    s = cache.struct()
    dev = cache.kv.device
    C = k_chunk.shape[2]
    _need(k_chunk, "k_chunk", (s.b, s.Hkv, C, s.d), cache.kv.dtype, dev)
    _need(v_chunk, "v_chunk", (s.b, s.Hkv, C, s.d), cache.kv.dtype, dev)
    _need(scores, "scores", (s.b, s.Hkv, C), torch.float32, dev)
    _need(quota, "quota", (s.b, s.Hkv), torch.int32, dev)
    if not workspace.is_contiguous() or workspace.device != dev:
        raise ValueError("workspace must be a contiguous tensor on the cache's device")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().kvs_prefill_chunk(ctypes.byref(s), _ptr(k_chunk), _ptr(v_chunk), _ptr(scores),
                                   _ptr(quota), int(C), _ptr(workspace), nbytes, _stream(stream)))


def kvs_prefill_quota(budgets: np.ndarray, contexts: np.ndarray, start: int,
                      chunk: int) -> np.ndarray:
    """[b][Hkv] int32 tokens each head keeps from prompt positions
    [start, start + chunk), for one layer's budgets [Hkv]."""
    B = np.ascontiguousarray(budgets, dtype=np.float64)
    N = np.ascontiguousarray(contexts, dtype=np.int64)
    if B.ndim != 1 or N.ndim != 1:
        raise ValueError("budgets [Hkv] and contexts [b] must be one-dimensional")
    q = np.zeros((N.shape[0], B.shape[0]), dtype=np.int32)
    _check(lib().kvs_prefill_quota(B.ctypes.data, N.ctypes.data, N.shape[0], B.shape[0],
                                   int(start), int(chunk), q.ctypes.data))
    return q


def kvs_rerank_heads(stable: np.ndarray, step: int, period: int) -> np.ndarray:
    """[Hkv] bool: the heads that re-select their pages at decode step ``step``."""
    st = np.ascontiguousarray(np.asarray(stable, dtype=bool).astype(np.uint8))
    if st.ndim != 1:
        raise ValueError("stable must be one-dimensional")
    due = np.zeros(st.shape[0], dtype=np.uint8)
    _check(lib().kvs_rerank_heads(st.ctypes.data, st.shape[0], int(step), int(period),
                                  due.ctypes.data))
    return due.astype(bool)


def kvs_plan_split(budgets: np.ndarray, head_slot: np.ndarray, Hp: int, cap: float,
                   T: int) -> np.ndarray:
    B = np.ascontiguousarray(budgets, dtype=np.float64)
    hs = np.ascontiguousarray(head_slot, dtype=np.int32)
    L, Hkv = B.shape
    S = np.zeros((L, Hkv // Hp), dtype=np.int32)
    _check(lib().kvs_plan_split(B.ctypes.data, hs.ctypes.data, L, Hkv, Hp, float(cap), int(T),
                                S.ctypes.data))
    return S


def kvs_cluster_heads(budgets: np.ndarray, Hp: int) -> np.ndarray:
    B = np.ascontiguousarray(budgets, dtype=np.float64)
    L, Hkv = B.shape
    hs = np.zeros((L, Hkv), dtype=np.int32)
    _check(lib().kvs_cluster_heads(B.ctypes.data, L, Hkv, Hp, hs.ctypes.data))
    return hs


def kvs_decode_workspace_bytes(b: int, Hq: int, Hkv: int, d: int, S_row: Sequence[int]) -> int:
    S = np.ascontiguousarray(S_row, dtype=np.int32)
    return int(lib().kvs_decode_workspace_bytes(b, Hq, Hkv, d, S.ctypes.data, len(S)))


def _decode_call(name: str, cache: Cache, q: torch.Tensor, sel: Optional[torch.Tensor],
                 sel_count: Optional[torch.Tensor], K: int, S_row: Sequence[int], scale: float,
                 workspace: torch.Tensor, out: torch.Tensor, stream) -> None:
    s = cache.struct()
    dev = cache.kv.device
    _need(q, "q", (s.b, s.Hq, s.d), cache.kv.dtype, dev)
    _need(out, "out", (s.b, s.Hq, s.d), torch.float32, dev)
    if sel is not None:
        _need(sel, "sel", (s.b, s.Hkv, K), torch.int32, dev)
        _need(sel_count, "sel_count", (s.b, s.Hkv), torch.int32, dev)
    if not workspace.is_contiguous() or workspace.device != dev:
        raise ValueError("workspace must be a contiguous tensor on the cache's device")
    S = np.ascontiguousarray(S_row, dtype=np.int32)
    if S.shape != (s.Hkv // s.Hp,):
        raise ValueError(f"S_row must have one entry per group ({s.Hkv // s.Hp})")
    nbytes = workspace.numel() * workspace.element_size()
    _check(getattr(lib(), name)(ctypes.byref(s), _ptr(q), _ptr(sel), _ptr(sel_count), int(K),
                                S.ctypes.data, float(scale), _ptr(workspace), nbytes, _ptr(out),
                                _stream(stream)))


def kvs_decode_attn(cache: Cache, q: torch.Tensor, sel: Optional[torch.Tensor],
                    sel_count: Optional[torch.Tensor], K: int, S_row: Sequence[int], scale: float,
                    workspace: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _decode_call("kvs_decode_attn", cache, q, sel, sel_count, K, S_row, scale, workspace, out,
                 stream)


def kvs_decode_splits(cache: Cache, q: torch.Tensor, sel: Optional[torch.Tensor],
                      sel_count: Optional[torch.Tensor], K: int, S_row: Sequence[int],
                      scale: float, workspace: torch.Tensor, out: torch.Tensor,
                      stream=None) -> None:
    """The split-K phase of kvs_decode_attn alone (partials into workspace)."""
    _decode_call("kvs_decode_splits", cache, q, sel, sel_count, K, S_row, scale, workspace, out,
                 stream)


def kvs_decode_combine(cache: Cache, q: torch.Tensor, sel: Optional[torch.Tensor],
                       sel_count: Optional[torch.Tensor], K: int, S_row: Sequence[int],
                       scale: float, workspace: torch.Tensor, out: torch.Tensor,
                       stream=None) -> None:
    """The combine phase of kvs_decode_attn alone (workspace partials into out)."""
    _decode_call("kvs_decode_combine", cache, q, sel, sel_count, K, S_row, scale, workspace, out,
                 stream)


# Bytes of scratch the library holds per device for kvs_decode_attn_noalloc.
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def kvs_decode_attn_noalloc(cache: Cache, q: torch.Tensor, sel: Optional[torch.Tensor],
                            sel_count: Optional[torch.Tensor], K: int, S_row: Sequence[int],
                            scale: float, out: torch.Tensor, stream=None) -> None:
    """kvs_decode_attn with the library's own per-device scratch instead of a
    workspace: allocates nothing.  Calls overlapping on one device race."""
    s = cache.struct()
    dev = cache.kv.device
    _need(q, "q", (s.b, s.Hq, s.d), cache.kv.dtype, dev)
    _need(out, "out", (s.b, s.Hq, s.d), torch.float32, dev)
    if sel is not None:
        _need(sel, "sel", (s.b, s.Hkv, K), torch.int32, dev)
        _need(sel_count, "sel_count", (s.b, s.Hkv), torch.int32, dev)
    S = np.ascontiguousarray(S_row, dtype=np.int32)
    if S.shape != (s.Hkv // s.Hp,):
        raise ValueError(f"S_row must have one entry per group ({s.Hkv // s.Hp})")
    _check(lib().kvs_decode_attn_noalloc(ctypes.byref(s), _ptr(q), _ptr(sel), _ptr(sel_count),
                                         int(K), S.ctypes.data, float(scale), _ptr(out),
                                         _stream(stream)))


def kvs_decode_concurrency(device: int, d: int, gqa: int, dtype: torch.dtype) -> int:
    W = ctypes.c_int32(0)
    _check(lib().kvs_decode_concurrency(device, d, gqa, dtype_code(dtype), ctypes.byref(W)))
    return W.value


def kvs_decode_stamps_offset(b: int, Hq: int, Hkv: int, d: int, S_row: Sequence[int]) -> int:
    """Instrumented build only: byte offset of the per-workgroup [start, end]
    uint64 stamps inside the decode workspace."""
    S = np.ascontiguousarray(S_row, dtype=np.int32)
    return int(lib().kvs_decode_stamps_offset(b, Hq, Hkv, d, S.ctypes.data, len(S)))


def kvs_score_stamps(dst: torch.Tensor, stream=None) -> None:
    """Instrumented build only: clock stamps [waves][3] (entry, share known,
    exit) of the last scoring launch into dst (int64 [waves][3])."""
    _check(lib().kvs_score_stamps(_ptr(dst), dst.shape[0], _stream(stream)))


def kvs_select_stamps(dst: torch.Tensor, stream=None) -> None:
    """Instrumented build only: clock stamps [blocks][12] (entry, up to
    eight waves' scoring done, past the barrier, K-th key known, exit) of the
    last one-launch selection."""
    _check(lib().kvs_select_stamps(_ptr(dst), dst.shape[0], _stream(stream)))
