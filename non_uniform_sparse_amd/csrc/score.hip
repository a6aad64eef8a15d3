// Quest-style page scores (FlexiCache summary, Core method): for a KV head h
// and page p, max over the query heads g of h of
//     sum_c max(q[g][c]*kmin[p][c], q[g][c]*kmax[p][c]).
// Since kmin <= kmax, the larger product is q*kmax when q >= 0 and q*kmin
// when q < 0, so each term is one pair-dot of q with a per-channel select of
// kmin/kmax driven by q's sign bits (equal values, one fewer product).
//
// One wave walks a chunk of 64 pages of one (request, head).  Lane l serves
// page l / COLS of each step and channels 8*(l % COLS) .. +8: two 16-byte
// loads (its kmin and kmax slices), fully coalesced per page.  Sums over a
// page's COLS lanes use a fixed butterfly, so results are deterministic.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kChunk = 64;   // pages per wave

template <int D, int GQ, typename DT>
__global__ __launch_bounds__(256) void score_kernel(CacheView c, const uint16_t* __restrict__ q,
                                                    float* __restrict__ scores) {
  constexpr int P = 16;
  constexpr int COLS = D / 8;
  constexpr int PPW = 64 / COLS;   // pages per step
  const int lane = threadIdx.x & 63;
  const int chunks = (c.maxpg + kChunk - 1) / kChunk;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= (int64_t)c.b * c.Hkv * chunks) return;
  const int chunk = (int)(wave % chunks);
  const int rh = (int)(wave / chunks);
  const int r = rh / c.Hkv, h = rh % c.Hkv;
  const int n = clampi(c.seq_len[rh], 0, P * c.maxpg);
  const int npg = (n + P - 1) / P;
  const int hs = c.head_slot[h];
  const bool head_ok = hs >= 0 && hs < c.Hkv;
  const int gi = head_ok ? hs / c.Hp : 0, slot = head_ok ? hs % c.Hp : 0;
  const int32_t* pt = c.page_table + ((int64_t)r * c.G + gi) * c.maxpg;

  const int pp = lane / COLS, col = lane % COLS;
  uint32_t qw[GQ][4], neg[GQ][4];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const uint4 v = ld16(q + ((int64_t)r * c.Hq + h * GQ + g) * D + 8 * col);
    qw[g][0] = v.x;
    qw[g][1] = v.y;
    qw[g][2] = v.z;
    qw[g][3] = v.w;
#pragma unroll
    for (int e = 0; e < 4; ++e) neg[g][e] = ((qw[g][e] & 0x80008000u) >> 15) * 0xffffu;
  }
  const uint16_t* mm = reinterpret_cast<const uint16_t*>(c.minmax);
  float* out = scores + (int64_t)rh * c.maxpg;

  for (int step = 0; step < kChunk / PPW; ++step) {
    const int p = chunk * kChunk + step * PPW + pp;
    int phys = -1;
    if (head_ok && p < npg) phys = pt[p];
    const bool live = phys >= 0 && phys < c.num_pages;
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (live) {
      const uint16_t* base = mm + ((int64_t)phys * c.Hp + slot) * 2 * D + 8 * col;
      lo = ld16(base);
      hi = ld16(base + D);
    }
    const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w};
    const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
    float best = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t pick = (hw[e] & ~neg[g][e]) | (lw[e] & neg[g][e]);
        acc = dot2(qw[g][e], pick, acc, DT());
      }
      acc = group_sum<COLS>(acc);
      best = fmaxf(best, acc);
    }
    if (col == 0 && p < c.maxpg) out[p] = live ? best : -__builtin_inff();
  }
}

template <int D, int GQ, typename DT>
hipError_t launch_v(const CacheView& c, const void* q, float* scores, hipStream_t s) {
  const int chunks = (c.maxpg + kChunk - 1) / kChunk;
  const int64_t waves = (int64_t)c.b * c.Hkv * chunks;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((score_kernel<D, GQ, DT>), dim3((unsigned)blocks), dim3(256), 0, s, c,
                     static_cast<const uint16_t*>(q), scores);
  return hipGetLastError();
}

template <int D, typename DT>
hipError_t launch_g(const CacheView& c, const void* q, float* scores, hipStream_t s) {
  switch (c.Gq) {
    case 1: return launch_v<D, 1, DT>(c, q, scores, s);
    case 2: return launch_v<D, 2, DT>(c, q, scores, s);
    case 4: return launch_v<D, 4, DT>(c, q, scores, s);
    default: return launch_v<D, 8, DT>(c, q, scores, s);
  }
}

}  // namespace

hipError_t launch_score(const CacheView& c, const void* q, float* scores, hipStream_t s) {
  if (c.dtype == KVS_F16)
    return c.d == 128 ? launch_g<128, F16>(c, q, scores, s) : launch_g<256, F16>(c, q, scores, s);
  return c.d == 128 ? launch_g<128, BF16>(c, q, scores, s) : launch_g<256, BF16>(c, q, scores, s);
}

}  // namespace kvs
