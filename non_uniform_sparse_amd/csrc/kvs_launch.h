// Launchers of libkvs's kernels other than the decode's, and the limits and
// argument bundles only they use.  Included by the entry points and by the
// sources that define these launchers.
#pragma once

#include "kvs_internal.h"

namespace kvs {

constexpr int kMaxChunk = 8192;          // prefill chunk length (16-bit kept positions)
constexpr int kMaxSlots = 1024;          // GPU pages per tiered head
constexpr int kMaxTierPages = 8192;      // max_group_pages of a tiered cache (LDS bitmap)

// A validated kvs_host_tier; host_kv is the device address of the pinned
// host pages.
struct HostTierView {
  void* host_kv;
  const int64_t* host_base;
  int32_t* slot_page;
  const int32_t* slot_phys;
  int slots;
  int64_t num_host_pages;
};

hipError_t launch_minmax(const CacheView& c, hipStream_t s);
hipError_t launch_score(const CacheView& c, const void* q, float* scores, const HeadMask& heads,
                        hipStream_t s);
hipError_t launch_topk(const float* scores, const int32_t* seq_len, int P, int b, int Hkv,
                       int max_pages, int K, const HeadMask& heads, int32_t* sel,
                       int32_t* sel_count, hipStream_t s);
hipError_t launch_select(const CacheView& c, const void* q, float* scores, int K, int32_t* sel,
                         int32_t* sel_count, hipStream_t s);
hipError_t launch_append(const CacheView& c, const HostTierView* tier, const void* k_new,
                         const void* v_new, hipStream_t s);
hipError_t launch_prefill(const CacheView& c, const void* k_chunk, const void* v_chunk,
                          const float* scores, const int32_t* quota, int C, void* ws,
                          hipStream_t s);
size_t prefill_workspace_bytes(int b, int Hkv, int C);
hipError_t launch_probe(const CacheView& c, const int32_t* sel, const int32_t* sel_count, int K,
                        uint32_t* sink, size_t sink_words, hipStream_t s);
int probe_sink_words(int d, int* words);
hipError_t launch_stream_probe(const void* src, size_t bytes, uint32_t* sink, size_t sink_words,
                               hipStream_t s);
int stream_probe_sink_words(int* words);
hipError_t launch_offload(const CacheView& c, const HostTierView& t, hipStream_t s);
hipError_t launch_promote(const CacheView& c, const HostTierView& t, const int32_t* sel,
                          const int32_t* sel_count, int K, const HeadMask& heads, int32_t* moved,
                          hipStream_t s);
// KV-cache codec: layout validation (shared by the encoder and the decoder)
// and the decode launch.
int codec_check_layout(const kvs_codec_layout* p, const char* fn);
hipError_t launch_codec_decode(const kvs_codec_layout& lay, const kvs_codec_chunk& ch, void* out,
                               hipStream_t s);

}  // namespace kvs
