// Device-side helpers shared by the gfx950 kernels: packed 16-bit element
// access, fp32-accumulating pair dot products and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvs_internal.h"

namespace kvs {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Element-type tags.  Both types are 16 bits wide; two elements are packed
// per 32-bit word, the lower-indexed element in the low half.
struct F16 {};
struct BF16 {};

// a.lo*b.lo + a.hi*b.hi + c with fp32 accumulation (v_dot2_f32_f16 /
// v_dot2_f32_bf16).  Products of 16-bit floats are exact in fp32.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, F16) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, BF16) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Low / high element of a packed word, widened to fp32 (exact).
__device__ __forceinline__ float lo_f(uint32_t v, F16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float hi_f(uint32_t v, F16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
__device__ __forceinline__ float lo_f(uint32_t v, BF16) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_f(uint32_t v, BF16) { return __uint_as_float(v & 0xffff0000u); }

// Narrow an fp32 value that is exactly representable in the 16-bit type.
__device__ __forceinline__ uint32_t narrow(float x, F16) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint32_t narrow(float x, BF16) { return __float_as_uint(x) >> 16; }

__device__ __forceinline__ uint32_t pack2(float lo, float hi, F16 t) {
  return narrow(lo, t) | (narrow(hi, t) << 16);
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi, BF16 t) {
  return narrow(lo, t) | (narrow(hi, t) << 16);
}

// Cross-lane moves without LDS.  DPP row patterns (a row is 16 lanes):
// quad_perm [1,0,3,2] = lane ^ 1, quad_perm [2,3,0,1] = lane ^ 2,
// row_half_mirror = 7 - (lane & 7), row_mirror = 15 - (lane & 15).
// v_permlane16_swap(x, x) returns {rows 0,0,2,2 ; rows 1,1,3,3} and
// v_permlane32_swap(x, x) returns {lanes 0-31 twice ; lanes 32-63 twice},
// so the sum of the pair is x + x[lane ^ 16] (resp. x[lane ^ 32]).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ void swap16(float v, float* a, float* b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  *a = __uint_as_float(r[0]);
  *b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float* a, float* b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  *a = __uint_as_float(r[0]);
  *b = __uint_as_float(r[1]);
}

// Sum / max over aligned groups of W lanes (W a power of two, 2..64).  Each
// level combines a lane with its partner in the other half of the group;
// once the values are uniform inside each half, mirror partners are as
// good as xor partners.  Every lane of a group ends with the same bitwise
// result: both partners combine the same two values.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W >= 2 && W <= 64 && (W & (W - 1)) == 0, "group width");
  v += dpp<0xB1>(v);
  if (W >= 4) v += dpp<0x4E>(v);
  if (W >= 8) v += dpp<0x141>(v);
  if (W >= 16) v += dpp<0x140>(v);
  if (W >= 32) {
    float a, b;
    swap16(v, &a, &b);
    v = a + b;
  }
  if (W >= 64) {
    float a, b;
    swap32(v, &a, &b);
    v = a + b;
  }
  return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
  static_assert(W >= 2 && W <= 64 && (W & (W - 1)) == 0, "group width");
  v = fmaxf(v, dpp<0xB1>(v));
  if (W >= 4) v = fmaxf(v, dpp<0x4E>(v));
  if (W >= 8) v = fmaxf(v, dpp<0x141>(v));
  if (W >= 16) v = fmaxf(v, dpp<0x140>(v));
  if (W >= 32) {
    float a, b;
    swap16(v, &a, &b);
    v = fmaxf(a, b);
  }
  if (W >= 64) {
    float a, b;
    swap32(v, &a, &b);
    v = fmaxf(a, b);
  }
  return v;
}
// Sum / max across lanes that differ only in lane bits >= FROM (FROM = 16
// or 32): combines the 64/FROM row groups holding the same columns.
template <int FROM>
__device__ __forceinline__ float across_sum(float v) {
  static_assert(FROM == 16 || FROM == 32, "across width");
  float a, b;
  if (FROM == 16) {
    swap16(v, &a, &b);
    v = a + b;
  }
  swap32(v, &a, &b);
  return a + b;
}
template <int FROM>
__device__ __forceinline__ float across_max(float v) {
  static_assert(FROM == 16 || FROM == 32, "across width");
  float a, b;
  if (FROM == 16) {
    swap16(v, &a, &b);
    v = fmaxf(a, b);
  }
  swap32(v, &a, &b);
  return fmaxf(a, b);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte load of data that is read once per pass (K/V tiles, page bounds):
// marked non-temporal, so the caches do not keep it at the expense of the
// data that is reused (page tables, queries, partials).
__device__ __forceinline__ uint4 ld16_once(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace kvs
