// Quest-style page scores (FlexiCache summary, Core method): for a KV head h
// and page p, max over the query heads g of h of
//     sum_c max(q[g][c]*kmin[p][c], q[g][c]*kmax[p][c]).
// Since kmin <= kmax, the larger product is q*kmax when q >= 0 and q*kmin
// when q < 0.  The metadata holds (min, max) per channel side by side, so
// for each channel pair one v_perm_b32 whose byte selector comes from q's
// sign bits picks the right bound of both channels, and one pair-dot adds
// the two products (equal values, one fewer product).
//
// One wave walks a chunk of 64 pages of one (request, head).  The chunk's
// physical page ids are fetched first, one per lane.  A page of one head is
// one contiguous 4*d-byte block, served by 8 lanes: load k of lane l reads
// 16 bytes (4 channels, both bounds) at quad 8k + l % 8 of page l / 8, so
// each load instruction reads one whole 128-byte line of each of 8 pages,
// and a page's sum is 3 DPP levels over its 8 lanes.  Steps (8 pages each)
// go in double-buffered rounds: the next round's loads are in flight while
// the current one is scored.  The butterfly order is fixed: deterministic.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kChunk = 64;   // pages per wave, one page id per lane

// Byte selector for v_perm_b32(b, a, sel) with a = (min_c, max_c) and
// b = (min_c1, max_c1): low half from a (max if q_c >= 0), high half from b.
__device__ __forceinline__ uint32_t pick_selector(uint32_t q_pair) {
  const bool pos0 = !(q_pair & 0x8000u), pos1 = !(q_pair & 0x80000000u);
  const uint32_t lo = pos0 ? 0x0302u : 0x0100u;
  const uint32_t hi = pos1 ? 0x0706u : 0x0504u;
  return lo | (hi << 16);
}

template <int D, int GQ, typename DT>
__global__ __launch_bounds__(256) void score_kernel(CacheView c, const uint16_t* __restrict__ q,
                                                    float* __restrict__ scores) {
  constexpr int P = 16;
  constexpr int LOADS = D / 32;           // 16-byte loads per lane per page
  constexpr int PPW = 8;                  // pages per step (8 lanes each)
  constexpr int STEPS = kChunk / PPW;     // 8
  constexpr int UNROLL = 16 / LOADS;      // steps per round: 64 data registers
  constexpr int ROUNDS = STEPS / UNROLL;
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

  const int pp = lane / 8, ql = lane % 8;   // page of the step, lane within the page
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
  const uint16_t* mm = reinterpret_cast<const uint16_t*>(c.minmax) + slot * 2 * D + 8 * ql;
  const int64_t page_stride = (int64_t)c.Hp * 2 * D;

  // Loads are unconditional (a missing page reads page 0 and is discarded),
  // which keeps the compiler's wait counting exact across the pipeline.
  uint4 mmv[2][UNROLL][LOADS];
  int live[2][UNROLL];
  auto issue = [&](int s0, uint4 (&dst)[UNROLL][LOADS], int (&ok)[UNROLL]) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int phys = __shfl(my_phys, (s0 + u) * PPW + pp, 64);
      ok[u] = phys >= 0;
      const uint16_t* base = mm + (phys >= 0 ? phys : 0) * page_stride;
#pragma unroll
      for (int k = 0; k < LOADS; ++k) dst[u][k] = ld16(base + 64 * k);
    }
  };
  auto score = [&](int s0, const uint4 (&src)[UNROLL][LOADS], const int (&ok)[UNROLL]) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float best = -__builtin_inff();
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < LOADS; ++k) {
          const uint4 w = src[u][k];
          acc = dot2(qw[g][k][0], __builtin_amdgcn_perm(w.y, w.x, sel[g][k][0]), acc, DT());
          acc = dot2(qw[g][k][1], __builtin_amdgcn_perm(w.w, w.z, sel[g][k][1]), acc, DT());
        }
        best = fmaxf(best, group_sum<8>(acc));
      }
      const int p = pbase + (s0 + u) * PPW + pp;
      if (ql == 0 && p < c.maxpg) out[p] = ok[u] ? best : -__builtin_inff();
    }
  };
  // two rounds per iteration so both buffers are named statically
  issue(0, mmv[0], live[0]);
  for (int rd = 0; rd < ROUNDS; rd += 2) {
    if (rd + 1 < ROUNDS) issue((rd + 1) * UNROLL, mmv[1], live[1]);
    score(rd * UNROLL, mmv[0], live[0]);
    if (rd + 1 < ROUNDS) {
      if (rd + 2 < ROUNDS) issue((rd + 2) * UNROLL, mmv[0], live[0]);
      score((rd + 1) * UNROLL, mmv[1], live[1]);
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
