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
// holds at once (one block per compute unit) and the pages are
// dealt out evenly: each block first forms
// the prefix sum of the heads' page counts in LDS (and copies the head-slot
// table there); wave w of W then takes flat pages [T*w/W, T*(w+1)/W) of the
// T in all heads, one segment per head it touches.
//
// A wave streams its share as one sequence of rounds (RP pages of one
// segment each) through a ring of two register buffers, across segment
// boundaries: the first round of the next head is loaded while the last
// round of the current head is scored, and a head's query rows are loaded
// before the following round is issued, so a head change costs no drained
// pipeline.  The next head's metadata base is fetched while the current
// segment streams.  Pages past a head's end get -inf from a final
// block-strided fill.
#include "flat_pages.h"
#include "kvs_launch.h"
#include "quest_bound.h"

namespace kvs {
namespace {

constexpr int kThreads = kFlatThreads;

// Pages of head rh to score: 0 for a head outside the set.
__device__ __forceinline__ int page_count(const CacheView& c, const HeadMask& heads, int rh) {
  constexpr int P = 16;
  if (!heads.has(rh % c.Hkv)) return 0;
  return (clampi(c.seq_len[rh], 0, P * c.maxpg) + P - 1) / P;
}

// The first head j >= from whose pages reach past flat page t (pre[j + 1] >
// t), 64 heads per probe; one exists when t < pre[BH] (else BH - 1).
__device__ __forceinline__ int next_head(const int* pre, int BH, int from, int t, int lane) {
  for (int j0 = from; j0 < BH; j0 += 64) {
    const int j = j0 + lane;
    const uint64_t hit = __ballot(j < BH && pre[min(j, BH - 1) + 1] > t);
    if (hit) return j0 + __builtin_ctzll(hit);
  }
  return BH - 1;
}

#ifdef KVS_WG_STAMPS
// Instrumented build only: per wave of the last scoring launch, the clock
// (s_memrealtime, 100 MHz) at entry, once its share is known, and at exit,
// each stored when taken.
constexpr int kScoreStampWaves = 16384;
__device__ uint64_t g_score_stamps[kScoreStampWaves][3];
#define KVS_SCORE_STAMP(k)                                                            \
  do {                                                                                \
    const int64_t w_ = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);    \
    if ((threadIdx.x & 63) == 0 && w_ < kScoreStampWaves)                             \
      g_score_stamps[w_][k] = __builtin_amdgcn_s_memrealtime();                       \
  } while (0)
#else
#define KVS_SCORE_STAMP(k) \
  do {                     \
  } while (0)
#endif

template <int D, int GQ, typename DT>
__global__ __launch_bounds__(kThreads) void score_kernel(CacheView c, const uint16_t* __restrict__ q,
                                                         float* __restrict__ scores, HeadMask heads) {
  constexpr int LOADS = D / 32;                          // 16-byte loads per lane per page
  constexpr int UNROLL = LOADS >= 8 ? 1 : 8 / LOADS;    // 8-page steps per round
  constexpr int RP = 8 * UNROLL;                         // pages per round
  extern __shared__ int pre[];
  __shared__ int part[kThreads];
  __shared__ int hslot[kMaxHkv];
  const int BH = c.b * c.Hkv;
  KVS_SCORE_STAMP(0);
  for (int i = threadIdx.x; i < c.Hkv; i += kThreads) hslot[i] = c.head_slot[i];
  page_prefix(BH, [&](int rh) { return page_count(c, heads, rh); }, pre, part);

  const int lane = threadIdx.x & 63;
  const int pp = lane / 8, ql = lane % 8;   // page of an 8-page step, lane within the page
  const FlatShare share = flat_share(pre, BH);
  KVS_SCORE_STAMP(1);
  const int t1 = share.t1;
  const int last = c.num_meta - 1;
  const uint16_t* mmb = reinterpret_cast<const uint16_t*>(c.minmax) + 8 * ql;

  // A segment: pages [p0, p1) of head rh, flat pages [base + p0, base + p1).
  struct Seg {
    int rh, base, p0, p1, mb, gi;
    bool ok;
  };
  auto make_seg = [&](int rh, int t, int mb) {
    Seg s;
    s.rh = rh;
    s.base = uni(pre[rh]);
    s.p0 = t - s.base;
    s.p1 = min(t1, uni(pre[rh + 1])) - s.base;
    s.mb = mb;
    const int hs = uni(hslot[rh % c.Hkv]);
    s.ok = hs >= 0 && hs < c.Hkv;
    s.gi = s.ok ? hs / c.Hp : 0;
    return s;
  };
  // Issue cursor: the round starting at page p of segment seg; the head
  // after seg (nx_rh, -1 if none) and its metadata base, fetched early.
  struct Cursor {
    Seg seg;
    int p;
    bool valid;
    int nx_rh, nx_mb;
  };
  auto fetch_next = [&](Cursor& k) {
    const int t = k.seg.base + k.seg.p1;
    k.nx_rh = t < t1 ? uni(next_head(pre, BH, k.seg.rh + 1, t, lane)) : -1;
    k.nx_mb = k.nx_rh >= 0 ? c.meta_base[k.nx_rh] : 0;
  };
  auto advance = [&](Cursor& k) {
    k.p += RP;
    if (k.p < k.seg.p1) return;
    if (k.nx_rh < 0) {
      k.valid = false;
      return;
    }
    k.seg = make_seg(k.nx_rh, k.seg.base + k.seg.p1, k.nx_mb);
    k.p = k.seg.p0;
    fetch_next(k);
  };
  // One issued round: its segment and first page.
  struct Slot {
    Seg seg;
    int p;
  };

  uint4 mmv[2][UNROLL][LOADS];
  int ptv[2][UNROLL];
  auto issue = [&](const Slot& s, uint4 (&dst)[UNROLL][LOADS], int (&pt)[UNROLL]) {
    const int r = s.seg.rh / c.Hkv;
    const int32_t* ptrow = c.page_table + ((int64_t)r * c.G + s.seg.gi) * c.maxpg;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int p = min(s.p + u * 8 + pp, s.seg.p1 - 1);
      int64_t m = (int64_t)s.seg.mb + p;
      m = m < 0 ? 0 : (m > last ? last : m);
      const uint16_t* bp = mmb + m * (2 * D);
#pragma unroll
      for (int k = 0; k < LOADS; ++k) dst[u][k] = ld16_once(bp + 64 * k);
      pt[u] = ptrow[p];
    }
  };
  QuestQuery<D, GQ> qq;
  int q_rh = -1;
  auto query_for = [&](const Slot& s) {   // before the next round is issued
    if (s.seg.rh == q_rh) return;
    const int r = s.seg.rh / c.Hkv, h = s.seg.rh - r * c.Hkv;
    qq.load(q + ((int64_t)r * c.Hq + h * GQ) * D, ql);
    q_rh = s.seg.rh;
  };
  auto score = [&](const Slot& s, const uint4 (&src)[UNROLL][LOADS], const int (&pt)[UNROLL]) {
    float* out = scores + (int64_t)s.seg.rh * c.maxpg;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const float best = qq.template bound<DT>(src[u]);
      const int p = s.p + u * 8 + pp;
      const int64_t m = (int64_t)s.seg.mb + p;
      const bool present = (pt[u] >= 0 && pt[u] < c.num_pages) || pt[u] == KVS_PAGE_ON_HOST;
      const bool ok = s.seg.ok && present && m >= 0 && m <= last;
      if (ql == 0 && p < s.seg.p1) out[p] = ok ? best : -__builtin_inff();
    }
  };

  if (share.t0 < t1) {
    Cursor cur;
    cur.seg = make_seg(share.hh, share.t0, c.meta_base[share.hh]);
    cur.p = cur.seg.p0;
    cur.valid = true;
    fetch_next(cur);
    Slot a{cur.seg, cur.p}, b;
    issue(a, mmv[0], ptv[0]);
    advance(cur);
    for (;;) {   // written out for two buffers: register indices stay static
      query_for(a);
      const bool more_b = cur.valid;
      if (more_b) {
        b = Slot{cur.seg, cur.p};
        issue(b, mmv[1], ptv[1]);
        advance(cur);
      }
      score(a, mmv[0], ptv[0]);
      if (!more_b) break;
      query_for(b);
      const bool more_a = cur.valid;
      if (more_a) {
        a = Slot{cur.seg, cur.p};
        issue(a, mmv[0], ptv[0]);
        advance(cur);
      }
      score(b, mmv[1], ptv[1]);
      if (!more_a) break;
    }
  }
  KVS_SCORE_STAMP(2);

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

// Blocks per compute unit at most.  A full resident grid (three blocks per
// unit at d = 256) scores a whole batch no faster than one, and in a step
// whose request micro-batches run on streams of their own, where score
// launches share the chip with the other parts' decode waves, one block per
// unit leaves those waves the most room and makes the whole step fastest.
// A small launch alone on the chip would stream faster with two.
constexpr int kScoreBlocksPerCu = 1;

template <int D, int GQ, typename DT>
hipError_t launch_v(const CacheView& c, const void* q, float* scores, const HeadMask& heads,
                    hipStream_t s) {
  int grid = 0;   // resident blocks, at most kScoreBlocksPerCu per compute unit
  if (hipError_t e = resident_grid<score_symbol<D, GQ, DT>>(&grid, kScoreBlocksPerCu)) return e;
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

#ifdef KVS_WG_STAMPS
hipError_t copy_score_stamps(uint64_t* dst, size_t waves, hipStream_t s) {
  void* src = nullptr;
  if (hipError_t e = hipGetSymbolAddress(&src, HIP_SYMBOL(g_score_stamps))) return e;
  if (waves > (size_t)kScoreStampWaves) waves = kScoreStampWaves;
  return hipMemcpyAsync(dst, src, waves * 3 * sizeof(uint64_t), hipMemcpyDeviceToDevice, s);
}
#endif

hipError_t launch_score(const CacheView& c, const void* q, float* scores, const HeadMask& heads,
                        hipStream_t s) {
  if (c.dtype == KVS_F16)
    return c.d == 128 ? launch_g<128, F16>(c, q, scores, heads, s)
                      : launch_g<256, F16>(c, q, scores, heads, s);
  return c.d == 128 ? launch_g<128, BF16>(c, q, scores, heads, s)
                    : launch_g<256, BF16>(c, q, scores, heads, s);
}

}  // namespace kvs
