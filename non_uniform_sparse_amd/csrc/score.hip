// Quest-style page scores (FlexiCache summary, Core method): for a KV head h
// and page p, max over the query heads g of h of
//     sum_c max(q[g][c]*kmin[p][c], q[g][c]*kmax[p][c]).
// Since kmin <= kmax, the larger product is q*kmax when q >= 0 and q*kmin
// when q < 0, so each term is one pair-dot of q with a per-channel select of
// kmin/kmax driven by q's sign bits (equal values, one fewer product).
//
// One wave walks a chunk of 64 pages of one (request, head).  The chunk's
// physical page ids are fetched first, one per lane, so the min-max loads of
// many steps can be in flight together (8 steps = 16 KB per wave).  Lane l
// serves page l / COLS of each step and channels 8*(l % COLS) .. +8: two
// 16-byte loads (its kmin and kmax slices), fully coalesced per page.  Sums
// over a page's COLS lanes use a fixed DPP butterfly: deterministic.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kChunk = 64;   // pages per wave, one page id per lane

template <int D, int GQ, typename DT>
__global__ __launch_bounds__(256) void score_kernel(CacheView c, const uint16_t* __restrict__ q,
                                                    float* __restrict__ scores) {
  constexpr int P = 16;
  constexpr int COLS = D / 8;
  constexpr int PPW = 64 / COLS;          // pages per step
  constexpr int STEPS = kChunk / PPW;
  constexpr int UNROLL = 8;
  static_assert(STEPS % UNROLL == 0, "unroll");
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
  const int pbase = chunk * kChunk;
  float* out = scores + (int64_t)rh * c.maxpg;

  // Physical id of page pbase + lane (-1 if absent or out of range).
  int my_phys = -1;
  if (head_ok && pbase + lane < npg) {
    my_phys = c.page_table[((int64_t)r * c.G + gi) * c.maxpg + pbase + lane];
    if (my_phys >= c.num_pages) my_phys = -1;
  }
  if (pbase >= npg) {   // nothing to score: pad with -inf
    if (pbase + lane < c.maxpg) out[pbase + lane] = -__builtin_inff();
    return;
  }

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
  const uint16_t* mm = reinterpret_cast<const uint16_t*>(c.minmax) + slot * 2 * D + 8 * col;
  const int64_t page_stride = (int64_t)c.Hp * 2 * D;

  for (int s0 = 0; s0 < STEPS; s0 += UNROLL) {
    uint4 lo[UNROLL], hi[UNROLL];
    int phys[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) phys[u] = __shfl(my_phys, (s0 + u) * PPW + pp, 64);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      lo[u] = make_uint4(0, 0, 0, 0);
      hi[u] = make_uint4(0, 0, 0, 0);
      if (phys[u] >= 0) {
        const uint16_t* base = mm + phys[u] * page_stride;
        lo[u] = ld16(base);
        hi[u] = ld16(base + D);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t lw[4] = {lo[u].x, lo[u].y, lo[u].z, lo[u].w};
      const uint32_t hw[4] = {hi[u].x, hi[u].y, hi[u].z, hi[u].w};
      float best = -__builtin_inff();
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t pick = (hw[e] & ~neg[g][e]) | (lw[e] & neg[g][e]);
          acc = dot2(qw[g][e], pick, acc, DT());
        }
        best = fmaxf(best, group_sum<COLS>(acc));
      }
      const int p = pbase + (s0 + u) * PPW + pp;
      if (col == 0 && p < c.maxpg) out[p] = phys[u] >= 0 ? best : -__builtin_inff();
    }
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
