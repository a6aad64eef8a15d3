// Quest-style page scores (FlexiCache summary, Core method): for a KV head h
// and page p, max over the query heads g of h of
//     sum_c max(q[g][c]*kmin[p][c], q[g][c]*kmax[p][c]),
// computed per page as quest_bound.h describes (one v_perm_b32 picks the
// bound each channel's sign needs, one pair-dot adds two channels, a fixed
// DPP butterfly sums a page's 8 lanes: deterministic).
//
// The work is a stream: every head's bounds are one contiguous run of
// 4*d-byte blocks (block meta_base[r][h] + p), and the read is bound by HBM.
// Heads differ widely in page count, so the grid is sized to what the chip
// holds at once and the pages are dealt out evenly: each block first forms
// the prefix sum of the heads' page counts in LDS; wave w of W then takes
// flat pages [T*w/W, T*(w+1)/W) of the T in all heads, which it walks as one
// segment per head it touches.  A segment loads its head's query rows once,
// then streams its pages in double-buffered rounds (score_run).  Pages past
// a head's end get -inf from a final block-strided fill.
#include "flat_pages.h"
#include "kvs_launch.h"
#include "quest_bound.h"

namespace kvs {
namespace {

constexpr int kThreads = kFlatThreads;
constexpr int kRing = 2;   // rounds of bounds per wave: one scored, one in flight

// Pages of head rh to score: 0 for a head outside the set.
__device__ __forceinline__ int page_count(const CacheView& c, const HeadMask& heads, int rh) {
  constexpr int P = 16;
  if (!heads.has(rh % c.Hkv)) return 0;
  return (clampi(c.seq_len[rh], 0, P * c.maxpg) + P - 1) / P;
}

template <int D, int GQ, typename DT>
__global__ __launch_bounds__(kThreads) void score_kernel(CacheView c, const uint16_t* __restrict__ q,
                                                         float* __restrict__ scores, HeadMask heads) {
  extern __shared__ int pre[];
  __shared__ int part[kThreads];
  const int BH = c.b * c.Hkv;
  page_prefix(BH, [&](int rh) { return page_count(c, heads, rh); }, pre, part);

  const int lane = threadIdx.x & 63;
  const int ql = lane % 8;   // lane within the page
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

    QuestQuery<D, GQ> qq;
    qq.load(q + ((int64_t)r * c.Hq + h * GQ) * D, ql);

    score_run<D, GQ, DT, kRing, 32>(qq, mmb, mb, last, ptrow, c.num_pages, head_ok, p0, p1, lane,
                         [&](int p, float v) { out[p] = v; });

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
