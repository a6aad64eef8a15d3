// Quest-style page scores (FlexiCache summary, Core method): for a KV head h
// and page p, max over the query heads g of h of
//     sum_c max(q[g][c]*kmin[p][c], q[g][c]*kmax[p][c]).
// Since kmin <= kmax, the larger product is q*kmax when q >= 0 and q*kmin
// when q < 0.  The metadata holds (min, max) per channel side by side, so
// for each channel pair one v_perm_b32 whose byte selector comes from q's
// sign bits picks the right bound of both channels, and one pair-dot adds
// the two products (equal values, one fewer product).
//
// The work is a stream: every head's bounds are one contiguous run of
// 4*d-byte blocks (block meta_base[r][h] + p), and the read is bound by HBM.
// Heads differ widely in page count, so the grid is sized to what the chip
// holds at once and the pages are dealt out evenly: each block first forms
// the prefix sum of the heads' page counts in LDS; wave w of W then takes
// flat pages [T*w/W, T*(w+1)/W) of the T in all heads, which it walks as one
// segment per head it touches.  A segment loads its head's query rows once,
// then streams rounds of pages: a page is served by 8 lanes, load k of lane
// l reading 16 bytes (4 channels, both bounds) at quad 8k + l % 8 of page
// l / 8, so each load instruction reads one whole 128-byte line of each of 8
// neighbouring pages, and a page's sum is 3 DPP levels over its 8 lanes.
// Rounds are double-buffered: the next round's loads are in flight while
// the current one is scored; no round past the segment's last is loaded
// (the test is uniform over the wave).  Inside a round the loads are
// unconditional: lanes past the segment's end read its last page again,
// within the same instructions.  The bounds are read with non-temporal loads
// (each is read once per pass).  The page table is read beside the
// bounds only to give null pages -inf; pages past a head's end get -inf
// from a final block-strided fill.  The butterfly order is fixed:
// deterministic.
#include "flat_pages.h"
#include "kvs_launch.h"

namespace kvs {
namespace {

constexpr int kThreads = kFlatThreads;

// Byte selector for v_perm_b32(b, a, sel) with a = (min_c, max_c) and
// b = (min_c1, max_c1): low half from a (max if q_c >= 0), high half from b.
__device__ __forceinline__ uint32_t pick_selector(uint32_t q_pair) {
  const bool pos0 = !(q_pair & 0x8000u), pos1 = !(q_pair & 0x80000000u);
  const uint32_t lo = pos0 ? 0x0302u : 0x0100u;
  const uint32_t hi = pos1 ? 0x0706u : 0x0504u;
  return lo | (hi << 16);
}

// Pages of head rh to score: 0 for a head outside the set.
__device__ __forceinline__ int page_count(const CacheView& c, const HeadMask& heads, int rh) {
  constexpr int P = 16;
  if (!heads.has(rh % c.Hkv)) return 0;
  return (clampi(c.seq_len[rh], 0, P * c.maxpg) + P - 1) / P;
}

template <int D, int GQ, typename DT>
__global__ __launch_bounds__(kThreads) void score_kernel(CacheView c, const uint16_t* __restrict__ q,
                                                         float* __restrict__ scores, HeadMask heads) {
  constexpr int LOADS = D / 32;           // 16-byte loads per lane per page
  constexpr int PPW = 8;                  // pages per step (8 lanes each)
  constexpr int UNROLL = 8 / LOADS > 0 ? 8 / LOADS : 1;   // steps per round: 32 data registers
  constexpr int RP = PPW * UNROLL;        // pages per round
  extern __shared__ int pre[];
  __shared__ int part[kThreads];
  const int BH = c.b * c.Hkv;
  page_prefix(BH, [&](int rh) { return page_count(c, heads, rh); }, pre, part);

  const int lane = threadIdx.x & 63;
  const int pp = lane / 8, ql = lane % 8;   // page of the step, lane within the page
  const FlatShare share = flat_share(pre, BH);
  int t0 = share.t0, hh = share.hh;
  const int t1 = share.t1;
  const int64_t last = c.num_meta - 1;
  const uint16_t* mmb = reinterpret_cast<const uint16_t*>(c.minmax) + 8 * ql;

  while (t0 < t1) {
    const int rh = hh;
    const int base = uni(pre[rh]);
    const int seg_end = min(t1, uni(pre[rh + 1]));
    const int p0 = t0 - base, p1 = seg_end - base;   // pages [p0, p1) of head rh
    const int r = rh / c.Hkv, h = rh - r * c.Hkv;
    const int hs = c.head_slot[h];
    const bool head_ok = hs >= 0 && hs < c.Hkv;
    const int gi = head_ok ? hs / c.Hp : 0;
    const int32_t* ptrow = c.page_table + ((int64_t)r * c.G + gi) * c.maxpg;
    const int64_t mb = c.meta_base[rh];
    float* out = scores + (int64_t)rh * c.maxpg;

    uint32_t qw[GQ][LOADS][2], sel[GQ][LOADS][2];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const uint16_t* qrow = q + ((int64_t)r * c.Hq + h * GQ + g) * D;
#pragma unroll
      for (int k = 0; k < LOADS; ++k) {
        const uint2 v = *reinterpret_cast<const uint2*>(qrow + 4 * (8 * k + ql));
        qw[g][k][0] = v.x;
        qw[g][k][1] = v.y;
        sel[g][k][0] = pick_selector(v.x);
        sel[g][k][1] = pick_selector(v.y);
      }
    }

    uint4 mmv[2][UNROLL][LOADS];
    int ptv[2][UNROLL];
    auto issue = [&](int rd, uint4 (&dst)[UNROLL][LOADS], int (&pt)[UNROLL]) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int p = min(p0 + rd * RP + u * PPW + pp, p1 - 1);
        int64_t m = mb + p;
        m = m < 0 ? 0 : (m > last ? last : m);
        const uint16_t* bp = mmb + m * (2 * D);
#pragma unroll
        for (int k = 0; k < LOADS; ++k) dst[u][k] = ld16_once(bp + 64 * k);
        pt[u] = ptrow[p];
      }
    };
    auto score = [&](int rd, const uint4 (&src)[UNROLL][LOADS], const int (&pt)[UNROLL]) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float best = -__builtin_inff();
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
          float acc = 0.f;
#pragma unroll
          for (int k = 0; k < LOADS; ++k) {
            const uint4 v = src[u][k];
            acc = dot2(qw[g][k][0], __builtin_amdgcn_perm(v.y, v.x, sel[g][k][0]), acc, DT());
            acc = dot2(qw[g][k][1], __builtin_amdgcn_perm(v.w, v.z, sel[g][k][1]), acc, DT());
          }
          best = fmaxf(best, group_sum<8>(acc));
        }
        const int p = p0 + rd * RP + u * PPW + pp;
        const int64_t m = mb + p;
        const bool present = (pt[u] >= 0 && pt[u] < c.num_pages) || pt[u] == KVS_PAGE_ON_HOST;
        const bool ok = head_ok && present && m >= 0 && m <= last;
        if (ql == 0 && p < p1) out[p] = ok ? best : -__builtin_inff();
      }
    };
    const int rounds = (p1 - p0 + RP - 1) / RP;
    issue(0, mmv[0], ptv[0]);
    for (int rd = 0; rd < rounds; rd += 2) {   // no round past the segment's last
      if (rd + 1 < rounds) issue(rd + 1, mmv[1], ptv[1]);
      score(rd, mmv[0], ptv[0]);
      if (rd + 2 < rounds) issue(rd + 2, mmv[0], ptv[0]);
      if (rd + 1 < rounds) score(rd + 1, mmv[1], ptv[1]);
    }

    t0 = seg_end;
    while (hh < BH && uni(pre[hh + 1]) <= t0) ++hh;
  }

  // -inf past each head's pages (heads outside the set keep their rows)
  for (int rh = blockIdx.x; rh < BH; rh += gridDim.x) {
    if (!heads.has(rh % c.Hkv)) continue;
    const int npg = pre[rh + 1] - pre[rh];
    float* out = scores + (int64_t)rh * c.maxpg;
    for (int p = npg + (int)threadIdx.x; p < c.maxpg; p += kThreads) out[p] = -__builtin_inff();
  }
}

template <int D, int GQ, typename DT>
const void* score_symbol() {
  return reinterpret_cast<const void*>(&score_kernel<D, GQ, DT>);
}

template <int D, int GQ, typename DT>
hipError_t launch_v(const CacheView& c, const void* q, float* scores, const HeadMask& heads,
                    hipStream_t s) {
  int grid = 0;   // one resident wave per slot
  if (hipError_t e = resident_grid<score_symbol<D, GQ, DT>>(&grid)) return e;
  const size_t lds = (size_t)(c.b * c.Hkv + 1) * sizeof(int);
  hipLaunchKernelGGL((score_kernel<D, GQ, DT>), dim3((unsigned)grid), dim3(kThreads), lds, s, c,
                     static_cast<const uint16_t*>(q), scores, heads);
  return hipGetLastError();
}

template <int D, typename DT>
hipError_t launch_g(const CacheView& c, const void* q, float* scores, const HeadMask& heads,
                    hipStream_t s) {
  switch (c.Gq) {
    case 1: return launch_v<D, 1, DT>(c, q, scores, heads, s);
    case 2: return launch_v<D, 2, DT>(c, q, scores, heads, s);
    case 4: return launch_v<D, 4, DT>(c, q, scores, heads, s);
    default: return launch_v<D, 8, DT>(c, q, scores, heads, s);
  }
}

}  // namespace

hipError_t launch_score(const CacheView& c, const void* q, float* scores, const HeadMask& heads,
                        hipStream_t s) {
  if (c.dtype == KVS_F16)
    return c.d == 128 ? launch_g<128, F16>(c, q, scores, heads, s)
                      : launch_g<256, F16>(c, q, scores, heads, s);
  return c.d == 128 ? launch_g<128, BF16>(c, q, scores, heads, s)
                    : launch_g<256, BF16>(c, q, scores, heads, s);
}

}  // namespace kvs
