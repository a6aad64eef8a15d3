// Internal declarations of libkvs shared by every kernel: limits, error
// reporting, the validated cache descriptor, head sets and the decode's
// argument bundle and launchers.  The other launchers are in kvs_launch.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvs.h"

namespace kvs {

constexpr int kMaxGroups = 64;     // G = Hkv / Hp
constexpr int kMaxHp = 16;         // heads per page group
constexpr int kMaxHkv = 128;
constexpr int kMaxTopkPages = 8192;
constexpr int kMaxK = 1024;
constexpr int kMaxSplitsPerRequest = 65536;
constexpr int kMaxScoreHeads = 16383;
constexpr float kLog2e = 1.4426950408889634f;

// Records a message for kvs_last_error() and returns `code`.
int set_error(int code, const char* fmt, ...);
void clear_error();

// A validated kvs_paged_kv with derived sizes.
struct CacheView {
  void* kv;
  void* minmax;
  const int32_t* meta_base;
  const int32_t* page_table;
  int32_t* seq_len;
  const int32_t* head_slot;
  int b, Hq, Hkv, Hp, G, Gq, d, P, maxpg, num_pages, num_meta, dtype;
};

// A set of KV heads, passed to kernels by value: every head, or the heads
// whose bit is set (bit h = head h, h < kMaxHkv).
struct HeadMask {
  uint32_t all;
  uint32_t w[kMaxHkv / 32];
  __host__ __device__ bool has(int h) const {
    return all != 0u || (h >= 0 && h < kMaxHkv && ((w[h >> 5] >> (h & 31)) & 1u));
  }
};

struct DecodeArgs {
  CacheView c;
  const void* q;
  const int32_t* sel;        // nullptr = every retained page
  const int32_t* sel_count;
  int K;
  float scale_log2;          // softmax scale * log2(e): logits kept in base 2
  float* o_part;             // [b][Hq][Smax][d]
  float* lse_part;           // [b][Hq][Smax], base-2 log-sum-exp
  int32_t* split_lo;         // [b][Hkv] first split touching each head
  int32_t* split_hi;         // [b][Hkv] last split touching each head
  uint64_t* stamps;          // instrumented build only: [b * splits_total][2] start/end
  int Smax;                  // max_i S_i
  int splits_total;          // sum_i S_i
  float* out;                // [b][Hq][d]
  int S_prefix[kMaxGroups + 1];
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine(const DecodeArgs& a, hipStream_t s);
// Resident decode workgroups per compute unit for a kernel variant.
hipError_t decode_blocks_per_cu(int d, int gqa, int dtype, int* blocks);

}  // namespace kvs
