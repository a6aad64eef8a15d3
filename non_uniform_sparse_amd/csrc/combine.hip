// Log-sum-exp combine of the split-K decode's partials (FlexiCache summary,
// Core method: flash-decoding merges each query head's split partials by
// their log-sum-exps):
//   out[r][g] = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max lse_s,
// over the splits s that touched the query head's KV head (base-2 lse, as
// the split kernel writes them).
#include <algorithm>

#include "decode_common.h"

namespace kvs {
namespace {

// Waves per combine workgroup at most.  Up to 16 merged a long-context
// layer's splits faster on their own, but in the micro-batched step such
// large workgroups wait for a compute unit the other parts' decode waves
// have left free, which gave a tail of slow steps; four keep the step's
// time tight.
constexpr int kCombineWaves = 4;

// One workgroup of W = blockDim.x / 64 waves (1 to 4) per (request, query
// head).  The splits that touched the head form the contiguous range
// [first, last] that the decode kernel recorded (an empty split inside it
// carries lse = -inf).  Wave w merges its W-th of the range, 8 splits per
// step: lane l takes split l / 8 of the step and channels (l % 8) * D/8 ..
// +D/8, and the wave keeps a running maximum m of the lse it has seen, its
// weighted sum and its total weight relative to m (a step that raises m
// rescales both first).  The loads of the next step are in flight while a
// step is merged, and no pass over the range precedes the merge.  The 8
// split lanes of each channel chunk are summed with DPP / lane swaps; the
// waves' (m, sum, weight) meet in LDS and are merged in wave order, so the
// result does not depend on timing.  A head spanning hundreds of splits
// (long, full-budget heads) is thus spread over up to 4 waves.
template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void combine_kernel(DecodeArgs a) {
  constexpr int CH = D / 8;          // channels per lane
  constexpr int V4 = CH / 4;         // float4 loads per split row
  constexpr int kMaxWaves = kCombineWaves;
  __shared__ float s_acc[kMaxWaves][D];
  __shared__ float s_m[kMaxWaves], s_den[kMaxWaves];
  const CacheView& c = a.c;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int r = blockIdx.x / c.Hq;
  const int g = blockIdx.x % c.Hq;
  const int h = g / c.Gq;
  const int64_t rh = (int64_t)r * c.Hkv + h;
  float* dst = a.out + ((int64_t)r * c.Hq + g) * D;
  // the head's unit count, exactly as the decode kernel forms it
  const int n = clampi(c.seq_len[rh], 0, P * c.maxpg);
  int cnt = (n + P - 1) / P;
  if (a.sel) cnt = min(cnt, clampi(a.sel_count[rh], 0, a.K));
  const int lo = a.split_lo[rh], hi = a.split_hi[rh];
  const int s_lo = cnt > 0 ? clampi(lo, 0, a.Smax - 1) : 0;
  const int s_hi = cnt > 0 ? clampi(hi, s_lo, a.Smax - 1) : -1;
  const int64_t row = ((int64_t)r * c.Hq + g) * a.Smax;
  // this wave's part of the range
  const int per = (s_hi - s_lo + 1 + W - 1) / W;
  const int w_lo = s_lo + wave * per, w_hi = min(s_hi, w_lo + per - 1);
  const int sl = lane / 8, dc = lane % 8;

  float acc[CH];
#pragma unroll
  for (int e = 0; e < CH; ++e) acc[e] = 0.f;
  float m = -__builtin_inff(), den = 0.f;
  // One step: the lse of split s0 + sl and its row slice (an in-bounds row
  // even past w_hi; such a lane's lse is -inf and its row is never used).
  auto load = [&](int s0, float& lse, float4 (&x)[V4]) {
    const int sp = s0 + sl;
    lse = sp <= w_hi ? a.lse_part[row + sp] : -__builtin_inff();
    const float4* src =
        reinterpret_cast<const float4*>(a.o_part + (row + min(sp, w_hi)) * D + dc * CH);
#pragma unroll
    for (int v = 0; v < V4; ++v) x[v] = src[v];
  };
  auto merge = [&](float lse, const float4 (&x)[V4]) {
    const float m_new = fmaxf(m, group_max<64>(lse));   // uniform over the wave
    if (!(m_new > -__builtin_inff())) return;           // nothing valid yet
    const float keep = m > -__builtin_inff() ? __builtin_amdgcn_exp2f(m - m_new) : 0.f;
    // an empty split (lse = -inf) weighs 0; its row may hold stale data, so
    // its contribution is selected away, never multiplied in
    const float wt = lse > -__builtin_inff() ? __builtin_amdgcn_exp2f(lse - m_new) : 0.f;
    const bool use = wt > 0.f;
    den = den * keep + wt;
#pragma unroll
    for (int v = 0; v < V4; ++v) {
      acc[4 * v] = acc[4 * v] * keep + (use ? wt * x[v].x : 0.f);
      acc[4 * v + 1] = acc[4 * v + 1] * keep + (use ? wt * x[v].y : 0.f);
      acc[4 * v + 2] = acc[4 * v + 2] * keep + (use ? wt * x[v].z : 0.f);
      acc[4 * v + 3] = acc[4 * v + 3] * keep + (use ? wt * x[v].w : 0.f);
    }
    m = m_new;
  };
  if (w_lo <= w_hi) {
    float l0, l1;
    float4 x0[V4], x1[V4];
    load(w_lo, l0, x0);
    for (int s0 = w_lo; s0 <= w_hi; s0 += 16) {   // no load past w_hi's step (uniform tests)
      if (s0 + 8 <= w_hi) load(s0 + 8, l1, x1);
      merge(l0, x0);
      if (s0 + 16 <= w_hi) load(s0 + 16, l0, x0);
      if (s0 + 8 <= w_hi) merge(l1, x1);
    }
  }
  // sums over the 8 split lanes of each channel chunk (lanes dc + 8 sl)
  den += dpp<0x128>(den);   // row_ror:8 -> lane ^ 8 within a row of 16
  den = across_sum<16>(den);
#pragma unroll
  for (int e = 0; e < CH; ++e) {
    float v = acc[e];
    v += dpp<0x128>(v);
    v = across_sum<16>(v);
    acc[e] = v;
  }
  if (W == 1) {   // one wave: its sums are the head's (uniform over the block)
    if (sl == 0) {
      const float inv = den > 0.f ? 1.f / den : 0.f;
      float4* o4 = reinterpret_cast<float4*>(dst + dc * CH);
#pragma unroll
      for (int v = 0; v < V4; ++v)
        o4[v] = make_float4(acc[4 * v] * inv, acc[4 * v + 1] * inv, acc[4 * v + 2] * inv,
                            acc[4 * v + 3] * inv);
    }
    return;
  }
  if (sl == 0) {
#pragma unroll
    for (int e = 0; e < CH; ++e) s_acc[wave][dc * CH + e] = acc[e];
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_den[wave] = den;
  }
  __syncthreads();
  // wave 0 merges the waves' sums in wave order, D / 64 channels per lane
  if (wave == 0) {
    float M = -__builtin_inff();
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w]);
    float dsum = 0.f, x[D / 64];
#pragma unroll
    for (int k = 0; k < D / 64; ++k) x[k] = 0.f;
    if (M > -__builtin_inff()) {
      for (int w = 0; w < W; ++w) {
        const float sc = s_m[w] > -__builtin_inff() ? __builtin_amdgcn_exp2f(s_m[w] - M) : 0.f;
        dsum += sc * s_den[w];
#pragma unroll
        for (int k = 0; k < D / 64; ++k) x[k] += sc * s_acc[w][lane + 64 * k];
      }
    }
    const float inv = dsum > 0.f ? 1.f / dsum : 0.f;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) dst[lane + 64 * k] = x[k] * inv;
  }
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.c.b * a.c.Hq;
  // one wave per 24 splits a head can span (a group's splits), at most
  // kCombineWaves
  const int waves = std::max(1, std::min(kCombineWaves, (a.Smax + 23) / 24));
  if (a.c.d == 128)
    hipLaunchKernelGGL((combine_kernel<128>), dim3((unsigned)blocks), dim3(64 * waves), 0, s, a);
  else
    hipLaunchKernelGGL((combine_kernel<256>), dim3((unsigned)blocks), dim3(64 * waves), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvs
