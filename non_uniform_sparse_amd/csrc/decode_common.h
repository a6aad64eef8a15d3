// Pieces of the split-K decode kernel: the unit bookkeeping of one
// (request, group) and the lane geometry and math of a page.
#pragma once

#include <utility>

#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int P = 16;

struct GroupUnits {
  int head[kMaxHp];    // KV head in each slot (-1 = empty slot)
  int count[kMaxHp];   // attended pages of each slot
  int start[kMaxHp];   // first unit of each slot
  int total;
};

// Heads and unit counts of group gi of request r.  Lane h reads head h's
// slot, length and selection count at once (no load waits on another), and
// the heads of group gi fill their slots' entries.
__device__ void group_units(const DecodeArgs& a, int r, int gi, GroupUnits* gu) {
  const CacheView& c = a.c;
  const int lane = threadIdx.x;
  if (lane < kMaxHp) {
    gu->head[lane] = -1;
    gu->count[lane] = 0;
  }
  __syncthreads();
  for (int h = lane; h < c.Hkv; h += 64) {
    const int hs = c.head_slot[h];
    const int n = clampi(c.seq_len[r * c.Hkv + h], 0, P * c.maxpg);
    const int sc = a.sel ? a.sel_count[r * c.Hkv + h] : 0;
    if (hs >= 0 && hs < c.Hkv && hs / c.Hp == gi) {
      int cnt = (n + P - 1) / P;
      if (a.sel) cnt = min(cnt, clampi(sc, 0, a.K));
      gu->head[hs % c.Hp] = h;
      gu->count[hs % c.Hp] = cnt;
    }
  }
  __syncthreads();
  if (lane == 0) {
    int acc = 0;
    for (int j = 0; j < c.Hp; ++j) {
      gu->start[j] = acc;
      acc += gu->count[j];
    }
    gu->total = acc;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Per-page math.  Logits of the page's 16 tokens against the GQ query heads
// form a small dense contraction, S^T[16 tokens][16 cols] = K[16][d] Q^T[d][16]
// (cols >= GQ are zero), done as d/32 v_mfma_f32_16x16x32 steps.  MFMA lane
// layouts (gfx950): A operand lane l holds A[l%16][8(l/16)..+8] of each 32-wide
// k block, B operand B[8(l/16)..+8][l%16], result D[4(l/16)+i][l%16], i < 4.
// MFMA row m is mapped to token tau(m) so that the result lands where the p*V
// step needs it: the V side gives lane l the channels 8*(l % COLS)..+8 of rows
// rg + RPL*k (rg = l / COLS, k < TL), and the result lane of column g in row
// group a = rg*A + hh (A = 4/RPL, hh < A) holds tokens rg + RPL*(4 hh + i).
// Softmax statistics live in the result layout (each lane tracks the query
// head of its column); probabilities and rescale factors reach the V lanes
// through ds_swizzle row broadcasts.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c, F16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c, BF16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ds_swizzle bit-mask mode within 32-lane halves: source = (lane & and) | or.
template <int AND, int OR>
__device__ __forceinline__ float swz(float v) {
  return __uint_as_float(__builtin_amdgcn_ds_swizzle(__float_as_uint(v), (OR << 5) | AND));
}

template <int D>
struct Geometry {
  static constexpr int COLS = D / 8;        // V lanes per row (8 channels each)
  static constexpr int RPL = 64 / COLS;     // V row groups
  static constexpr int TL = P / RPL;        // rows per V lane
  static constexpr int A = 4 / RPL;         // result row groups per V row group
  static constexpr int KB = D / 32;         // MFMA k blocks
};

// Value held by result lane (row group rg*A + HH, column G) broadcast to every
// lane of V row group rg.
template <int D, int HH, int G>
__device__ __forceinline__ float from_result(float v) {
  constexpr int A = Geometry<D>::A;
  if constexpr (A == 1) return swz<0x10, G>(v);      // rows of 16; keep lane bit 4
  else return swz<0x00, 16 * HH + G>(v);             // two result rows per 32-lane half
}

}  // namespace
}  // namespace kvs
