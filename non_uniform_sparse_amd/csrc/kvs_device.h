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

// Butterfly reductions over aligned lane groups of width W (a power of two,
// W <= 64).  Every lane of a group ends with the same, bitwise identical,
// result: at each level both partners add the same two partial values.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
// Reduce across lanes that differ in the bits >= FROM (lane ^ FROM, lane ^ 2*FROM, ...).
template <int FROM>
__device__ __forceinline__ float across_sum(float v) {
#pragma unroll
  for (int m = FROM; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}
template <int FROM>
__device__ __forceinline__ float across_max(float v) {
#pragma unroll
  for (int m = FROM; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace kvs
