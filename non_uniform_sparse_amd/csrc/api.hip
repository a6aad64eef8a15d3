// C-ABI entry points of libkvs: argument validation (before any HIP call),
// error reporting, workspace sizing and the kernel launches.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kvs_internal.h"
#include "kvs_launch.h"

namespace kvs {

namespace {
thread_local char g_err[512] = "";

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hip_error(hipError_t e, const char* what) {
  return set_error(KVS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Validates the cache descriptor.  need_minmax: the call reads or writes it.
int check_cache(const kvs_paged_kv* p, bool need_minmax, const char* fn, CacheView* v) {
  if (!p) return set_error(KVS_EINVAL, "%s: cache descriptor is NULL", fn);
  if (!p->kv || !p->page_table || !p->seq_len || !p->head_slot ||
      (need_minmax && (!p->minmax || !p->meta_base)))
    return set_error(KVS_EINVAL, "%s: null device pointer in cache descriptor", fn);
  if (need_minmax && p->num_meta < 1)
    return set_error(KVS_EINVAL, "%s: num_meta must be positive", fn);
  if (!aligned16(p->kv) || (need_minmax && !aligned16(p->minmax)))
    return set_error(KVS_EINVAL, "%s: kv and minmax must be 16-byte aligned", fn);
  if (p->b < 1 || p->Hkv < 1 || p->Hq < 1 || p->Hp < 1 || p->max_group_pages < 1 ||
      p->num_pages < 1)
    return set_error(KVS_EINVAL, "%s: sizes must be positive", fn);
  if (p->Hq % p->Hkv) return set_error(KVS_EINVAL, "%s: Hq %% Hkv != 0", fn);
  if (p->Hkv % p->Hp) return set_error(KVS_EINVAL, "%s: Hkv %% Hp != 0", fn);
  if (p->Hkv > kMaxHkv || p->Hp > kMaxHp || p->Hkv / p->Hp > kMaxGroups)
    return set_error(KVS_EUNSUPPORTED, "%s: need Hkv <= %d, Hp <= %d, G <= %d", fn, kMaxHkv,
                     kMaxHp, kMaxGroups);
  const int gq = p->Hq / p->Hkv;
  if (gq != 1 && gq != 2 && gq != 4 && gq != 8)
    return set_error(KVS_EUNSUPPORTED, "%s: query group size %d not in {1,2,4,8}", fn, gq);
  if (p->d != 128 && p->d != 256)
    return set_error(KVS_EUNSUPPORTED, "%s: head_dim %d not in {128, 256}", fn, p->d);
  if (p->P != 16) return set_error(KVS_EUNSUPPORTED, "%s: page size %d != 16", fn, p->P);
  if (p->dtype != KVS_F16 && p->dtype != KVS_BF16)
    return set_error(KVS_EUNSUPPORTED, "%s: dtype %d is neither f16 nor bf16", fn, p->dtype);
  if ((int64_t)p->b * p->Hkv * p->max_group_pages > ((int64_t)1 << 40) ||
      (int64_t)p->P * p->max_group_pages > 0x7fffffff)
    return set_error(KVS_EINVAL, "%s: cache too large", fn);
  v->kv = p->kv;
  v->minmax = p->minmax;
  v->meta_base = p->meta_base;
  v->num_meta = p->num_meta;
  v->page_table = p->page_table;
  v->seq_len = p->seq_len;
  v->head_slot = p->head_slot;
  v->b = p->b;
  v->Hq = p->Hq;
  v->Hkv = p->Hkv;
  v->Hp = p->Hp;
  v->G = p->Hkv / p->Hp;
  v->Gq = gq;
  v->d = p->d;
  v->P = p->P;
  v->maxpg = p->max_group_pages;
  v->num_pages = p->num_pages;
  v->dtype = p->dtype;
  return KVS_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Partial outputs, log-sum-exps, then each head's split range:
// [b][Hq][Smax][d] f32, [b][Hq][Smax] f32, [b][Hkv] i32 (first), [b][Hkv] i32 (last).
size_t workspace_bytes(int b, int Hq, int Hkv, int d, int Smax) {
  const size_t rows = (size_t)b * Hq * Smax;
  return round256(rows * d * sizeof(float)) + round256(rows * sizeof(float)) +
         2 * round256((size_t)b * Hkv * sizeof(int32_t));
}

#ifdef KVS_WG_STAMPS
// Instrumented build: per-workgroup start/end stamps follow the workspace.
size_t stamp_bytes(int b, int splits_total) { return round256((size_t)b * splits_total * 16); }
#endif

}  // namespace

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

}  // namespace kvs

using namespace kvs;

extern "C" const char* kvs_last_error(void) { return g_err; }

extern "C" int kvs_build_minmax(const kvs_paged_kv* cache, void* stream) {
  clear_error();
  CacheView c;
  if (int rc = check_cache(cache, true, "kvs_build_minmax", &c)) return rc;
  if ((int64_t)c.b * c.Hkv > kMaxScoreHeads)   // the heads' page counts are scanned in LDS
    return set_error(KVS_EUNSUPPORTED, "kvs_build_minmax: b*Hkv > %d", kMaxScoreHeads);
  if (hipError_t e = launch_minmax(c, (hipStream_t)stream)) return hip_error(e, "kvs_build_minmax");
  return KVS_OK;
}

namespace {
HeadMask every_head() {
  HeadMask m{};
  m.all = 1u;
  return m;
}

// The heads h < Hkv with heads[h] != 0 (host array), or an error.
int head_subset(const uint8_t* heads, int Hkv, HeadMask* m, const char* fn) {
  if (!heads) return set_error(KVS_EINVAL, "%s: heads is NULL", fn);
  if (Hkv > kMaxHkv) return set_error(KVS_EUNSUPPORTED, "%s: Hkv=%d > %d", fn, Hkv, kMaxHkv);
  *m = HeadMask{};
  for (int h = 0; h < Hkv; ++h)
    if (heads[h]) m->w[h >> 5] |= 1u << (h & 31);
  return KVS_OK;
}

int score_impl(const kvs_paged_kv* cache, const void* q, float* scores, const HeadMask& heads,
               void* stream, const char* fn) {
  CacheView c;
  if (int rc = check_cache(cache, true, fn, &c)) return rc;
  if (!q || !scores) return set_error(KVS_EINVAL, "%s: null q or scores", fn);
  if (!aligned16(q)) return set_error(KVS_EINVAL, "%s: q must be 16-byte aligned", fn);
  if ((int64_t)c.b * c.Hkv > kMaxScoreHeads)
    return set_error(KVS_EUNSUPPORTED, "%s: b*Hkv=%lld > %d", fn, (long long)c.b * c.Hkv,
                     kMaxScoreHeads);
  if ((int64_t)c.b * c.Hkv * c.maxpg > 0x7fffffff)
    return set_error(KVS_EUNSUPPORTED, "%s: b*Hkv*max_group_pages >= 2^31", fn);
  if (hipError_t e = launch_score(c, q, scores, heads, (hipStream_t)stream)) return hip_error(e, fn);
  return KVS_OK;
}

int topk_impl(const float* scores, const int32_t* seq_len, int32_t P, int32_t b, int32_t Hkv,
              int32_t max_pages, int32_t K, const HeadMask& heads, int32_t* sel,
              int32_t* sel_count, void* stream, const char* fn) {
  if (!scores || !seq_len || !sel || !sel_count) return set_error(KVS_EINVAL, "%s: null pointer", fn);
  if (P != 16) return set_error(KVS_EUNSUPPORTED, "%s: page size %d != 16", fn, P);
  if (b < 1 || Hkv < 1 || max_pages < 1)
    return set_error(KVS_EINVAL, "%s: sizes must be positive", fn);
  if (K < 1 || K > kMaxK) return set_error(KVS_EINVAL, "%s: K=%d not in [1, %d]", fn, K, kMaxK);
  if (max_pages > kMaxTopkPages)
    return set_error(KVS_EUNSUPPORTED, "%s: max_pages=%d > %d", fn, max_pages, kMaxTopkPages);
  if ((int64_t)b * Hkv > 0x7fffffff) return set_error(KVS_EINVAL, "%s: b*Hkv too large", fn);
  if (hipError_t e = launch_topk(scores, seq_len, P, b, Hkv, max_pages, K, heads, sel, sel_count,
                                 (hipStream_t)stream))
    return hip_error(e, fn);
  return KVS_OK;
}
}  // namespace

extern "C" int kvs_score_pages(const kvs_paged_kv* cache, const void* q, float* scores,
                               void* stream) {
  clear_error();
  return score_impl(cache, q, scores, every_head(), stream, "kvs_score_pages");
}

extern "C" int kvs_score_pages_heads(const kvs_paged_kv* cache, const void* q,
                                     const uint8_t* heads, float* scores, void* stream) {
  clear_error();
  static const char* fn = "kvs_score_pages_heads";
  if (!cache) return set_error(KVS_EINVAL, "%s: cache descriptor is NULL", fn);
  HeadMask m;
  if (int rc = head_subset(heads, cache->Hkv, &m, fn)) return rc;
  return score_impl(cache, q, scores, m, stream, fn);
}

extern "C" int kvs_topk_pages(const float* scores, const int32_t* seq_len, int32_t P, int32_t b,
                              int32_t Hkv, int32_t max_pages, int32_t K, int32_t* sel,
                              int32_t* sel_count, void* stream) {
  clear_error();
  return topk_impl(scores, seq_len, P, b, Hkv, max_pages, K, every_head(), sel, sel_count, stream,
                   "kvs_topk_pages");
}

extern "C" int kvs_topk_pages_heads(const float* scores, const int32_t* seq_len, int32_t P,
                                    int32_t b, int32_t Hkv, int32_t max_pages, int32_t K,
                                    const uint8_t* heads, int32_t* sel, int32_t* sel_count,
                                    void* stream) {
  clear_error();
  static const char* fn = "kvs_topk_pages_heads";
  HeadMask m;
  if (int rc = head_subset(heads, Hkv, &m, fn)) return rc;
  return topk_impl(scores, seq_len, P, b, Hkv, max_pages, K, m, sel, sel_count, stream, fn);
}

extern "C" int kvs_select_pages(const kvs_paged_kv* cache, const void* q, float* scores,
                                int32_t K, int32_t* sel, int32_t* sel_count, void* stream) {
  clear_error();
  static const char* fn = "kvs_select_pages";
  CacheView c;
  if (int rc = check_cache(cache, true, fn, &c)) return rc;
  if (!q || !sel || !sel_count) return set_error(KVS_EINVAL, "%s: null q, sel or sel_count", fn);
  if (!aligned16(q)) return set_error(KVS_EINVAL, "%s: q must be 16-byte aligned", fn);
  if (K < 1 || K > kMaxK) return set_error(KVS_EINVAL, "%s: K=%d not in [1, %d]", fn, K, kMaxK);
  if (c.maxpg > kMaxTopkPages)
    return set_error(KVS_EUNSUPPORTED, "%s: max_group_pages=%d > %d", fn, c.maxpg, kMaxTopkPages);
  if ((int64_t)c.b * c.Hkv * c.maxpg > 0x7fffffff)
    return set_error(KVS_EUNSUPPORTED, "%s: b*Hkv*max_group_pages >= 2^31", fn);
  if (hipError_t e = launch_select(c, q, scores, K, sel, sel_count, (hipStream_t)stream))
    return hip_error(e, fn);
  return KVS_OK;
}

extern "C" size_t kvs_prefill_workspace_bytes(int32_t b, int32_t Hkv, int32_t C) {
  if (b < 1 || Hkv < 1 || C < 1 || C > kMaxChunk) return 0;
  return prefill_workspace_bytes(b, Hkv, C);
}

extern "C" int kvs_prefill_chunk(const kvs_paged_kv* cache, const void* k_chunk,
                                 const void* v_chunk, const float* scores, const int32_t* quota,
                                 int32_t C, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  static const char* fn = "kvs_prefill_chunk";
  CacheView c;
  if (int rc = check_cache(cache, true, fn, &c)) return rc;
  if (!k_chunk || !v_chunk || !scores || !quota)
    return set_error(KVS_EINVAL, "%s: null chunk, scores or quota", fn);
  if (!aligned16(k_chunk) || !aligned16(v_chunk))
    return set_error(KVS_EINVAL, "%s: k_chunk and v_chunk must be 16-byte aligned", fn);
  if (C < 1 || C > kMaxChunk)
    return set_error(KVS_EINVAL, "%s: chunk length %d not in [1, %d]", fn, C, kMaxChunk);
  if ((int64_t)c.b * c.Hkv > 65535) return set_error(KVS_EUNSUPPORTED, "%s: b*Hkv > 65535", fn);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return set_error(KVS_EINVAL, "%s: workspace must be non-null and 256-byte aligned", fn);
  const size_t need = prefill_workspace_bytes(c.b, c.Hkv, C);
  if (ws_bytes < need)
    return set_error(KVS_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  if (hipError_t e = launch_prefill(c, k_chunk, v_chunk, scores, quota, C, workspace,
                                    (hipStream_t)stream))
    return hip_error(e, fn);
  return KVS_OK;
}

extern "C" int kvs_append_kv(const kvs_paged_kv* cache, const void* k_new, const void* v_new,
                             void* stream) {
  clear_error();
  static const char* fn = "kvs_append_kv";
  CacheView c;
  if (int rc = check_cache(cache, true, fn, &c)) return rc;
  if (!k_new || !v_new) return set_error(KVS_EINVAL, "%s: null k_new or v_new", fn);
  if (!aligned16(k_new) || !aligned16(v_new))
    return set_error(KVS_EINVAL, "%s: k_new and v_new must be 16-byte aligned", fn);
  if (hipError_t e = launch_append(c, nullptr, k_new, v_new, (hipStream_t)stream))
    return hip_error(e, fn);
  return KVS_OK;
}

extern "C" int kvs_gather_probe_sink_words(int32_t d, int32_t* words) {
  clear_error();
  if (!words || (d != 128 && d != 256))
    return set_error(KVS_EINVAL, "kvs_gather_probe_sink_words: null output or head_dim not 128/256");
  if (probe_sink_words(d, words))
    return set_error(KVS_EHIP, "kvs_gather_probe_sink_words: occupancy query failed");
  return KVS_OK;
}

extern "C" int kvs_gather_probe(const kvs_paged_kv* cache, const int32_t* sel,
                                const int32_t* sel_count, int32_t K, uint32_t* sink,
                                size_t sink_words, void* stream) {
  clear_error();
  static const char* fn = "kvs_gather_probe";
  CacheView c;
  if (int rc = check_cache(cache, false, fn, &c)) return rc;
  if (!sink) return set_error(KVS_EINVAL, "%s: null sink", fn);
  if ((sel == nullptr) != (sel_count == nullptr))
    return set_error(KVS_EINVAL, "%s: sel and sel_count go together", fn);
  if (sel && (K < 1 || K > kMaxK)) return set_error(KVS_EINVAL, "%s: K=%d not in [1, %d]", fn, K, kMaxK);
  if ((int64_t)c.b * c.Hkv > kMaxScoreHeads)
    return set_error(KVS_EUNSUPPORTED, "%s: b*Hkv > %d", fn, kMaxScoreHeads);
  if (hipError_t e = launch_probe(c, sel, sel_count, K, sink, sink_words, (hipStream_t)stream))
    return e == hipErrorInvalidValue ? set_error(KVS_ENOSPC, "%s: sink too small", fn)
                                     : hip_error(e, fn);
  return KVS_OK;
}

extern "C" int kvs_stream_probe_sink_words(int32_t* words) {
  clear_error();
  if (!words) return set_error(KVS_EINVAL, "kvs_stream_probe_sink_words: null output");
  if (stream_probe_sink_words(words))
    return set_error(KVS_EHIP, "kvs_stream_probe_sink_words: occupancy query failed");
  return KVS_OK;
}

extern "C" int kvs_stream_probe(const void* src, size_t bytes, uint32_t* sink, size_t sink_words,
                                void* stream) {
  clear_error();
  static const char* fn = "kvs_stream_probe";
  if (!src || !sink) return set_error(KVS_EINVAL, "%s: null src or sink", fn);
  if (!aligned16(src) || (bytes & 15) || bytes == 0)
    return set_error(KVS_EINVAL, "%s: src 16-byte aligned, bytes a positive multiple of 16", fn);
  if (hipError_t e = launch_stream_probe(src, bytes, sink, sink_words, (hipStream_t)stream))
    return e == hipErrorInvalidValue ? set_error(KVS_ENOSPC, "%s: sink too small", fn)
                                     : hip_error(e, fn);
  return KVS_OK;
}

extern "C" int kvs_codec_decode(const kvs_codec_layout* layout, const kvs_codec_chunk* chunk,
                                void* out, void* stream) {
  clear_error();
  static const char* fn = "kvs_codec_decode";
  if (int rc = codec_check_layout(layout, fn)) return rc;
  if (!chunk || !out) return set_error(KVS_EINVAL, "%s: null chunk or output", fn);
  if (!chunk->lo || !chunk->scale || !chunk->tab_first || !chunk->tab_n || !chunk->tab_off ||
      !chunk->cdf || !chunk->streams || !chunk->stream_off || chunk->cdf_len < 1 ||
      chunk->streams_len < 8)
    return set_error(KVS_EINVAL, "%s: null pointer, empty table pool or streams in chunk", fn);
  if (!aligned16(out)) return set_error(KVS_EINVAL, "%s: out must be 16-byte aligned", fn);
  if (reinterpret_cast<uintptr_t>(chunk->streams) & 3)
    return set_error(KVS_EINVAL, "%s: streams must be 4-byte aligned", fn);
  if (hipError_t e = launch_codec_decode(*layout, *chunk, out, (hipStream_t)stream))
    return hip_error(e, fn);
  return KVS_OK;
}

namespace {
// Validates the host tier of a cache: first the descriptor's fields, then
// (the one HIP call, made after every other check of the entry point) that
// host_kv is pinned host memory mapped for the current device, whose device
// address goes to the kernels.
int check_tier_fields(const kvs_host_tier* p, const CacheView& c, const char* fn) {
  if (!p) return set_error(KVS_EINVAL, "%s: tier descriptor is NULL", fn);
  if (!p->host_kv || !p->host_base || !p->slot_page || !p->slot_phys)
    return set_error(KVS_EINVAL, "%s: null pointer in tier descriptor", fn);
  if (c.Hp != 1) return set_error(KVS_EUNSUPPORTED, "%s: a host tier needs Hp == 1", fn);
  if (p->slots < 1 || p->slots > kMaxSlots)
    return set_error(KVS_EINVAL, "%s: slots=%d not in [1, %d]", fn, p->slots, kMaxSlots);
  if (p->num_host_pages < 1 || p->num_host_pages > 0x7fffffff)
    return set_error(KVS_EINVAL, "%s: num_host_pages not in [1, 2^31)", fn);
  if (!aligned16(p->host_kv)) return set_error(KVS_EINVAL, "%s: host_kv must be 16-byte aligned", fn);
  return KVS_OK;
}

int map_tier(const kvs_host_tier* p, const char* fn, HostTierView* t) {
  hipPointerAttribute_t a;
  const hipError_t e = hipPointerGetAttributes(&a, p->host_kv);
  if (e != hipSuccess) {
    (void)hipGetLastError();   // leave no error behind for the caller's next call
    return set_error(KVS_EINVAL, "%s: host_kv is not memory known to HIP (%s)", fn,
                     hipGetErrorString(e));
  }
  if (a.type != hipMemoryTypeHost || !a.devicePointer)
    return set_error(KVS_EINVAL, "%s: host_kv is not pinned host memory mapped for the device",
                     fn);
  t->host_kv = a.devicePointer;
  t->host_base = p->host_base;
  t->slot_page = p->slot_page;
  t->slot_phys = p->slot_phys;
  t->slots = p->slots;
  t->num_host_pages = p->num_host_pages;
  return KVS_OK;
}
}  // namespace

extern "C" int kvs_offload_pages(const kvs_paged_kv* cache, const kvs_host_tier* tier,
                                 void* stream) {
  clear_error();
  static const char* fn = "kvs_offload_pages";
  CacheView c;
  if (int rc = check_cache(cache, false, fn, &c)) return rc;
  if ((int64_t)c.b * c.Hkv > 65535) return set_error(KVS_EUNSUPPORTED, "%s: b*Hkv > 65535", fn);
  if (int rc = check_tier_fields(tier, c, fn)) return rc;
  HostTierView t;
  if (int rc = map_tier(tier, fn, &t)) return rc;
  if (hipError_t e = launch_offload(c, t, (hipStream_t)stream)) return hip_error(e, fn);
  return KVS_OK;
}

extern "C" int kvs_append_kv_tier(const kvs_paged_kv* cache, const kvs_host_tier* tier,
                                  const void* k_new, const void* v_new, void* stream) {
  clear_error();
  static const char* fn = "kvs_append_kv_tier";
  CacheView c;
  if (int rc = check_cache(cache, true, fn, &c)) return rc;
  if (!k_new || !v_new) return set_error(KVS_EINVAL, "%s: null k_new or v_new", fn);
  if (!aligned16(k_new) || !aligned16(v_new))
    return set_error(KVS_EINVAL, "%s: k_new and v_new must be 16-byte aligned", fn);
  if (int rc = check_tier_fields(tier, c, fn)) return rc;
  HostTierView t;
  if (int rc = map_tier(tier, fn, &t)) return rc;
  if (hipError_t e = launch_append(c, &t, k_new, v_new, (hipStream_t)stream)) return hip_error(e, fn);
  return KVS_OK;
}

extern "C" int kvs_promote_pages(const kvs_paged_kv* cache, const kvs_host_tier* tier,
                                 const int32_t* sel, const int32_t* sel_count, int32_t K,
                                 const uint8_t* heads, int32_t* moved, void* stream) {
  clear_error();
  static const char* fn = "kvs_promote_pages";
  CacheView c;
  if (int rc = check_cache(cache, false, fn, &c)) return rc;
  if (!sel || !sel_count) return set_error(KVS_EINVAL, "%s: null sel or sel_count", fn);
  if (c.maxpg > kMaxTierPages)
    return set_error(KVS_EUNSUPPORTED, "%s: max_group_pages=%d > %d", fn, c.maxpg, kMaxTierPages);
  if ((int64_t)c.b * c.Hkv > 0x7fffffff) return set_error(KVS_EINVAL, "%s: b*Hkv too large", fn);
  if (int rc = check_tier_fields(tier, c, fn)) return rc;
  if (K < 1 || K > tier->slots)
    return set_error(KVS_EINVAL, "%s: K=%d not in [1, slots=%d]", fn, K, tier->slots);
  HeadMask m = every_head();
  if (heads && head_subset(heads, c.Hkv, &m, fn)) return KVS_EINVAL;
  HostTierView t;
  if (int rc = map_tier(tier, fn, &t)) return rc;
  if (hipError_t e = launch_promote(c, t, sel, sel_count, K, m, moved, (hipStream_t)stream))
    return hip_error(e, fn);
  return KVS_OK;
}

namespace {
// Checks S_row and fills the split prefix sums; returns Smax via *smax.
int check_splits(const int32_t* S_row, int G, int b, DecodeArgs* a, int* smax, const char* fn) {
  if (!S_row) return set_error(KVS_EINVAL, "%s: S_row is NULL", fn);
  int64_t acc = 0;
  int mx = 0;
  a->S_prefix[0] = 0;
  for (int i = 0; i < G; ++i) {
    if (S_row[i] < 1) return set_error(KVS_EINVAL, "%s: S_row[%d]=%d < 1", fn, i, S_row[i]);
    acc += S_row[i];
    if (acc > kMaxSplitsPerRequest)
      return set_error(KVS_EINVAL, "%s: sum(S_row) > %d", fn, kMaxSplitsPerRequest);
    a->S_prefix[i + 1] = (int)acc;
    mx = S_row[i] > mx ? S_row[i] : mx;
  }
  if ((int64_t)b * acc > 0x7fffffff) return set_error(KVS_EINVAL, "%s: too many workgroups", fn);
  a->splits_total = (int)acc;
  *smax = mx;
  return KVS_OK;
}
}  // namespace

extern "C" size_t kvs_decode_workspace_bytes(int32_t b, int32_t Hq, int32_t Hkv, int32_t d,
                                             const int32_t* S_row, int32_t G) {
  if (b < 1 || Hq < 1 || Hkv < 1 || d < 1 || G < 1 || G > kMaxGroups || !S_row) return 0;
  DecodeArgs a;
  int smax = 0;
  if (check_splits(S_row, G, b, &a, &smax, "kvs_decode_workspace_bytes")) return 0;
#ifdef KVS_WG_STAMPS
  return workspace_bytes(b, Hq, Hkv, d, smax) + stamp_bytes(b, a.splits_total);
#else
  return workspace_bytes(b, Hq, Hkv, d, smax);
#endif
}

namespace {
// Validates the decode's arguments other than the workspace, fills *a (all
// but the workspace pointers) and the workspace bytes it needs.
int decode_prepare(const kvs_paged_kv* cache, const void* q, const int32_t* sel,
                   const int32_t* sel_count, int32_t K, const int32_t* S_row, float scale,
                   float* out, const char* fn, DecodeArgs* a, size_t* need, size_t* stamps_at) {
  memset(a, 0, sizeof *a);
  if (int rc = check_cache(cache, false, fn, &a->c)) return rc;
  if (!q || !out) return set_error(KVS_EINVAL, "%s: null q or out", fn);
  if (!aligned16(q) || !aligned16(out))
    return set_error(KVS_EINVAL, "%s: q and out need 16-byte alignment", fn);
  if (sel && (!sel_count || K < 1 || K > kMaxK))
    return set_error(KVS_EINVAL, "%s: with sel, need sel_count and 1 <= K <= %d", fn, kMaxK);
  if (!(scale > 0.f) || !(scale < 1e30f)) return set_error(KVS_EINVAL, "%s: bad scale", fn);
  int smax = 0;
  if (int rc = check_splits(S_row, a->c.G, a->c.b, a, &smax, fn)) return rc;
  *need = workspace_bytes(a->c.b, a->c.Hq, a->c.Hkv, a->c.d, smax);
  *stamps_at = *need;
#ifdef KVS_WG_STAMPS
  *need += stamp_bytes(a->c.b, a->splits_total);
#endif
  a->q = q;
  a->sel = sel;
  a->sel_count = sel_count;
  a->K = sel ? K : 0;
  a->scale_log2 = scale * kLog2e;
  a->Smax = smax;
  a->out = out;
  return KVS_OK;
}

// Which kernels decode_launch runs.
enum : int { kSplitPhase = 1, kCombinePhase = 2, kBothPhases = 3 };

// Carves the workspace (256-byte aligned, large enough) and launches the
// split kernel, the combine, or both.
int decode_launch(DecodeArgs& a, void* workspace, size_t stamps_at, hipStream_t s,
                  int phases = kBothPhases) {
  char* ws = static_cast<char*>(workspace);
  const size_t rows = (size_t)a.c.b * a.c.Hq * a.Smax;
  a.o_part = reinterpret_cast<float*>(ws);
  ws += round256(rows * a.c.d * sizeof(float));
  a.lse_part = reinterpret_cast<float*>(ws);
  ws += round256(rows * sizeof(float));
  a.split_lo = reinterpret_cast<int32_t*>(ws);
  ws += round256((size_t)a.c.b * a.c.Hkv * sizeof(int32_t));
  a.split_hi = reinterpret_cast<int32_t*>(ws);
#ifdef KVS_WG_STAMPS
  a.stamps = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + stamps_at);
#else
  (void)stamps_at;
#endif
  if (phases & kSplitPhase)
    if (hipError_t e = launch_decode(a, s)) return hip_error(e, "decode (split kernel)");
  if (phases & kCombinePhase)
    if (hipError_t e = launch_combine(a, s)) return hip_error(e, "decode (combine kernel)");
  return KVS_OK;
}

// kvs_decode_attn, kvs_decode_splits and kvs_decode_combine: the same
// checks, then the phases asked for.
int decode_entry(const kvs_paged_kv* cache, const void* q, const int32_t* sel,
                 const int32_t* sel_count, int32_t K, const int32_t* S_row, float scale,
                 void* workspace, size_t ws_bytes, float* out, void* stream, const char* fn,
                 int phases) {
  clear_error();
  DecodeArgs a;
  size_t need = 0, stamps_at = 0;
  if (int rc = decode_prepare(cache, q, sel, sel_count, K, S_row, scale, out, fn, &a, &need,
                              &stamps_at))
    return rc;
  if (!workspace || ((uintptr_t)workspace & 255u))
    return set_error(KVS_EINVAL, "%s: workspace must be non-null and 256-byte aligned", fn);
  if (ws_bytes < need)
    return set_error(KVS_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  return decode_launch(a, workspace, stamps_at, (hipStream_t)stream, phases);
}
}  // namespace

extern "C" int kvs_decode_attn(const kvs_paged_kv* cache, const void* q, const int32_t* sel,
                               const int32_t* sel_count, int32_t K, const int32_t* S_row,
                               float scale, void* workspace, size_t ws_bytes, float* out,
                               void* stream) {
  return decode_entry(cache, q, sel, sel_count, K, S_row, scale, workspace, ws_bytes, out, stream,
                      "kvs_decode_attn", kBothPhases);
}

extern "C" int kvs_decode_splits(const kvs_paged_kv* cache, const void* q, const int32_t* sel,
                                 const int32_t* sel_count, int32_t K, const int32_t* S_row,
                                 float scale, void* workspace, size_t ws_bytes, float* out,
                                 void* stream) {
  return decode_entry(cache, q, sel, sel_count, K, S_row, scale, workspace, ws_bytes, out, stream,
                      "kvs_decode_splits", kSplitPhase);
}

extern "C" int kvs_decode_combine(const kvs_paged_kv* cache, const void* q, const int32_t* sel,
                                  const int32_t* sel_count, int32_t K, const int32_t* S_row,
                                  float scale, void* workspace, size_t ws_bytes, float* out,
                                  void* stream) {
  return decode_entry(cache, q, sel, sel_count, K, S_row, scale, workspace, ws_bytes, out, stream,
                      "kvs_decode_combine", kCombinePhase);
}

// ---------------------------------------------------------------------------
// kvs_decode_attn without a caller workspace, for callers that cannot
// allocate device memory.  Its scratch is this file-scope device array:
// every device the library runs on holds its own copy, from the first use
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory, so the host never passes it to a kernel: the device
// address of each device's copy comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KVS_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_of[kMaxScratchDevices];

// The current device's copy of `scratch` (its address looked up once).
int noalloc_scratch(void** ptr, const char* fn) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return hip_error(e, fn);
  if (dev < 0 || dev >= kMaxScratchDevices)
    return set_error(KVS_EUNSUPPORTED, "%s: device %d >= %d", fn, dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_of[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return hip_error(e, fn);
    if (!p || ((uintptr_t)p & 255u))
      return set_error(KVS_EHIP, "%s: no aligned device address for the scratch array", fn);
    g_scratch_of[dev] = p;
  }
  *ptr = g_scratch_of[dev];
  return KVS_OK;
}
}  // namespace

extern "C" int kvs_decode_attn_noalloc(const kvs_paged_kv* cache, const void* q,
                                       const int32_t* sel, const int32_t* sel_count, int32_t K,
                                       const int32_t* S_row, float scale, float* out,
                                       void* stream) {
  clear_error();
  const char* fn = "kvs_decode_attn_noalloc";
  DecodeArgs a;
  size_t need = 0, stamps_at = 0;
  if (int rc = decode_prepare(cache, q, sel, sel_count, K, S_row, scale, out, fn, &a, &need,
                              &stamps_at))
    return rc;
  if (need > (size_t)KVS_NOALLOC_SCRATCH_BYTES)
    return set_error(KVS_ENOSPC,
                     "%s: this shape and split row need %zu bytes of scratch, more than the "
                     "%zu the library holds per device; use kvs_decode_attn with a workspace",
                     fn, need, (size_t)KVS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int rc = noalloc_scratch(&ws, fn)) return rc;
  return decode_launch(a, ws, stamps_at, (hipStream_t)stream);
}

extern "C" int kvs_decode_concurrency(int32_t device, int32_t d, int32_t gqa, int32_t dtype,
                                      int32_t* W) {
  clear_error();
  const char* fn = "kvs_decode_concurrency";
  if (!W) return set_error(KVS_EINVAL, "%s: W is NULL", fn);
  if (d != 128 && d != 256) return set_error(KVS_EUNSUPPORTED, "%s: head_dim %d", fn, d);
  if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8)
    return set_error(KVS_EUNSUPPORTED, "%s: query group size %d", fn, gqa);
  if (dtype != KVS_F16 && dtype != KVS_BF16)
    return set_error(KVS_EUNSUPPORTED, "%s: dtype %d", fn, dtype);
  int cus = 0, blocks = 0;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device))
    return hip_error(e, fn);
  if (hipError_t e = decode_blocks_per_cu(d, gqa, dtype, &blocks)) return hip_error(e, fn);
  *W = cus * blocks;
  return KVS_OK;
}

#ifdef KVS_WG_STAMPS
namespace kvs {
hipError_t copy_score_stamps(uint64_t* dst, size_t waves, hipStream_t s);
hipError_t copy_select_stamps(uint64_t* dst, size_t blocks, hipStream_t s);
}
// Instrumented build only: the [blocks][12] uint64 clock stamps (entry, each
// of up to eight waves' scoring done, past the barrier, K-th key known,
// exit) of the last one-launch selection's first `blocks` workgroups, copied
// to dst (device).
extern "C" int kvs_select_stamps(uint64_t* dst, size_t blocks, void* stream) {
  clear_error();
  if (!dst) return set_error(KVS_EINVAL, "kvs_select_stamps: null dst");
  if (hipError_t e = copy_select_stamps(dst, blocks, (hipStream_t)stream))
    return hip_error(e, "kvs_select_stamps");
  return KVS_OK;
}
// Instrumented build only: the [waves][3] uint64 clock stamps (entry, share
// known, exit) of the last scoring launch's first `waves` waves, copied to
// dst (device) on `stream`.
extern "C" int kvs_score_stamps(uint64_t* dst, size_t waves, void* stream) {
  clear_error();
  if (!dst) return set_error(KVS_EINVAL, "kvs_score_stamps: null dst");
  if (hipError_t e = copy_score_stamps(dst, waves, (hipStream_t)stream))
    return hip_error(e, "kvs_score_stamps");
  return KVS_OK;
}

// Instrumented build only: byte offset of the [b * sum(S_row)][2] uint64
// start/end stamps (s_memrealtime, 100 MHz) inside the decode workspace.
extern "C" size_t kvs_decode_stamps_offset(int32_t b, int32_t Hq, int32_t Hkv, int32_t d,
                                           const int32_t* S_row, int32_t G) {
  if (b < 1 || Hq < 1 || Hkv < 1 || d < 1 || G < 1 || G > kMaxGroups || !S_row) return 0;
  DecodeArgs a;
  int smax = 0;
  if (check_splits(S_row, G, b, &a, &smax, "kvs_decode_stamps_offset")) return 0;
  return workspace_bytes(b, Hq, Hkv, d, smax);
}
#endif
