// The Quest page bound of one KV head (FlexiCache summary, Core method), as
// eight lanes of a wave compute it for one page: shared by the scoring kernel
// and the fused score + top-K kernel, so that both produce the same bits.
//
// For query row g and page p the bound is sum_c max(q[g][c]*kmin[p][c],
// q[g][c]*kmax[p][c]); since kmin <= kmax the larger product is q*kmax when
// q >= 0 and q*kmin otherwise.  The metadata holds (min, max) per channel side
// by side, so for each channel pair one v_perm_b32 whose byte selector comes
// from q's sign bits picks the right bound of both channels, and one pair-dot
// adds the two products.  Lane ql of the page's eight holds the channel
// quads 8k + ql (k < D/32) of the query rows and of the page's bounds; the
// eight lanes' sums meet in a fixed DPP butterfly, and the head's bound is
// the max over its query rows.
#pragma once

#include "kvs_device.h"

namespace kvs {
namespace {

// Byte selector for v_perm_b32(b, a, sel) with a = (min_c, max_c) and
// b = (min_c1, max_c1): low half from a (max if q_c >= 0), high half from b.
__device__ __forceinline__ uint32_t pick_selector(uint32_t q_pair) {
  const bool pos0 = !(q_pair & 0x8000u), pos1 = !(q_pair & 0x80000000u);
  const uint32_t lo = pos0 ? 0x0302u : 0x0100u;
  const uint32_t hi = pos1 ? 0x0706u : 0x0504u;
  return lo | (hi << 16);
}

// The head's query rows in lane ql's layout, and their selectors.
template <int D, int GQ>
struct QuestQuery {
  static constexpr int LOADS = D / 32;   // 16-byte loads per lane per page
  uint32_t qw[GQ][LOADS][2], sel[GQ][LOADS][2];
  __device__ __forceinline__ void load(const uint16_t* q_head, int ql) {
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const uint16_t* qrow = q_head + (int64_t)g * D;
#pragma unroll
      for (int k = 0; k < LOADS; ++k) {
        const uint2 v = *reinterpret_cast<const uint2*>(qrow + 4 * (8 * k + ql));
        qw[g][k][0] = v.x;
        qw[g][k][1] = v.y;
        sel[g][k][0] = pick_selector(v.x);
        sel[g][k][1] = pick_selector(v.y);
      }
    }
  }
  // The page's bound from this lane's LOADS bound words; every lane of the
  // page's eight returns it.
  template <typename DT>
  __device__ __forceinline__ float bound(const uint4 (&src)[LOADS]) const {
    float best = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < LOADS; ++k) {
        const uint4 v = src[k];
        acc = dot2(qw[g][k][0], __builtin_amdgcn_perm(v.y, v.x, sel[g][k][0]), acc, DT());
        acc = dot2(qw[g][k][1], __builtin_amdgcn_perm(v.w, v.z, sel[g][k][1]), acc, DT());
      }
      best = fmaxf(best, group_sum<8>(acc));
    }
    return best;
  }
};

// Scores pages [p0, p1) of one head and calls emit(p, score) once per page,
// on the page's lane ql == 0.  Lane l serves page l / 8 of each step of 8
// pages, load k of its lane reading 16 bytes (4 channels, both bounds) at
// quad 8k + l % 8, so each load instruction reads one whole 128-byte line of
// each of 8 neighbouring pages.  Rounds of RP pages go through a ring of NB
// register buffers: the next NB - 1 rounds' loads are in flight while the
// current one is scored, and no round past the last is loaded (the test is
// uniform over the wave); inside
// a round the loads are unconditional and lanes past p1 read page p1 - 1
// again, within the same instructions.  The bounds are read with
// non-temporal loads (each is read once per pass).  The page table is read
// beside the bounds only to give null pages -inf.
//   mmb     minmax + 8 * ql (elements), the lane's quad of block 0
//   mb      the head's first metadata block; last: the highest valid block
//   ptrow   the page-table row of the head's group
//   NB      round buffers; DATA: data registers per round buffer
template <int D, int GQ, typename DT, int NB, int DATA, typename Emit>
__device__ __forceinline__ void score_run(const QuestQuery<D, GQ>& qq, const uint16_t* mmb,
                                          int64_t mb, int64_t last, const int32_t* ptrow,
                                          int num_pages, bool head_ok, int p0, int p1, int lane,
                                          Emit emit) {
  constexpr int LOADS = D / 32;
  constexpr int PPW = 8;                                  // pages per step (8 lanes each)
  constexpr int UNROLL = DATA / (4 * LOADS) > 0 ? DATA / (4 * LOADS) : 1;   // steps per round
  constexpr int RP = PPW * UNROLL;                        // pages per round
  const int pp = lane / 8, ql = lane % 8;
  uint4 mmv[NB][UNROLL][LOADS];
  int ptv[NB][UNROLL];
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
      const float best = qq.template bound<DT>(src[u]);
      const int p = p0 + rd * RP + u * PPW + pp;
      const int64_t m = mb + p;
      const bool present = (pt[u] >= 0 && pt[u] < num_pages) || pt[u] == KVS_PAGE_ON_HOST;
      const bool ok = head_ok && present && m >= 0 && m <= last;
      if (ql == 0 && p < p1) emit(p, ok ? best : -__builtin_inff());
    }
  };
  const int rounds = (p1 - p0 + RP - 1) / RP;
  if (rounds <= 0) return;
  if constexpr (NB == 2) {   // written out: the compiler keeps the loads' waits tighter
    issue(0, mmv[0], ptv[0]);
    for (int rd = 0; rd < rounds; rd += 2) {
      if (rd + 1 < rounds) issue(rd + 1, mmv[1], ptv[1]);
      score(rd, mmv[0], ptv[0]);
      if (rd + 2 < rounds) issue(rd + 2, mmv[0], ptv[0]);
      if (rd + 1 < rounds) score(rd + 1, mmv[1], ptv[1]);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j + 1 < NB; ++j)
    if (j < rounds) issue(j, mmv[j], ptv[j]);
  for (int rd = 0; rd < rounds; rd += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {   // round rd + j sits in buffer j
      const int nx = rd + j + NB - 1;
      if (nx < rounds) issue(nx, mmv[(j + NB - 1) % NB], ptv[(j + NB - 1) % NB]);
      if (rd + j < rounds) score(rd + j, mmv[j], ptv[j]);
    }
  }
}

}  // namespace
}  // namespace kvs
