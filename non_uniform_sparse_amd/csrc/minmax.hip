// Min-max page metadata builder (FlexiCache summary, Key observations,
// assumption 2: per-page key bounds kept on the GPU, apart from the KV pages).
//
// Every valid page of every head is read once, so the build is a stream of
// K tiles bound by HBM.  The grid is resident-sized and each wave takes an
// even share of all heads' pages (flat_pages.h), walking it as one segment
// per head.  A segment resolves the physical ids of 64 pages at a time
// (lane-parallel), then streams their K tiles two at a time: the next
// page's tile is in flight while the current one is reduced.  A page's K
// tile is P = 16 rows of d contiguous elements; lane l reads 16 bytes (8
// channels) of rows rg + RPL*k, rg = l / COLS, so each load instruction
// covers RPL whole rows (1 KB).  Per-channel min/max over the lane's rows,
// then across the RPL row groups with lane swaps.  The output is
// channel-interleaved, (min, max) per channel, so that one page of one head
// is a single contiguous 4*d-byte block, and goes to block meta_base[r][h] +
// p of the min-max cache, not to the page's physical KV slot: each head's
// bounds form one contiguous run in page order.  Loads are unconditional (a
// missing page reads page 0 and is discarded; indices are clamped into the
// segment), which keeps the compiler's wait counting exact.
#include "flat_pages.h"
#include "kvs_launch.h"

namespace kvs {
namespace {

__device__ __forceinline__ int head_pages(const CacheView& c, int rh) {
  constexpr int P = 16;
  return (clampi(c.seq_len[rh], 0, P * c.maxpg) + P - 1) / P;
}

template <int D, typename DT>
__global__ __launch_bounds__(kFlatThreads) void minmax_kernel(CacheView c) {
  constexpr int P = 16;
  constexpr int COLS = D / 8;      // lanes per row
  constexpr int RPL = 64 / COLS;   // rows per load
  constexpr int TL = P / RPL;      // rows per lane
  extern __shared__ int pre[];
  __shared__ int part[kFlatThreads];
  const int BH = c.b * c.Hkv;
  page_prefix(BH, [&](int rh) { return head_pages(c, rh); }, pre, part);

  const int lane = threadIdx.x & 63;
  const int rg = lane / COLS, col = lane % COLS;
  const FlatShare share = flat_share(pre, BH);
  int t0 = share.t0, hh = share.hh;
  const int t1 = share.t1;
  const uint16_t* kvb = reinterpret_cast<const uint16_t*>(c.kv) + rg * D + 8 * col;
  const int64_t last_meta = c.num_meta - 1;

  while (t0 < t1) {
    const int rh = hh;
    const int base = uni(pre[rh]);
    const int seg_end = min(t1, uni(pre[rh + 1]));
    const int p0 = t0 - base, p1 = seg_end - base;   // pages [p0, p1) of head rh
    const int r = rh / c.Hkv, h = rh - r * c.Hkv;
    const int n = clampi(c.seq_len[rh], 0, P * c.maxpg);
    const int hs = c.head_slot[h];
    const bool head_ok = hs >= 0 && hs < c.Hkv;
    const int gi = head_ok ? hs / c.Hp : 0, slot = head_ok ? hs % c.Hp : 0;
    const int32_t* ptrow = c.page_table + ((int64_t)r * c.G + gi) * c.maxpg;
    const int64_t mb = c.meta_base[rh];

    for (int b0 = p0; b0 < p1; b0 += 64) {
      const int nb = min(64, p1 - b0);
      // physical id of page b0 + lane (-1: absent, null or out of range)
      int my_phys = ptrow[b0 + min(lane, nb - 1)];
      if (!head_ok || lane >= nb || my_phys >= c.num_pages) my_phys = -1;
      auto tile = [&](int i) {
        const int phys = __builtin_amdgcn_readlane(my_phys, i);
        return kvb + (phys >= 0 ? ((int64_t)phys * c.Hp + slot) * 2 * P * D : 0);
      };
      auto load = [&](const uint16_t* t, uint4 (&dst)[TL]) {
#pragma unroll
        for (int k = 0; k < TL; ++k) dst[k] = ld16(t + RPL * k * D);
      };
      auto reduce_store = [&](int i, const uint4 (&src)[TL]) {
        const int phys = __builtin_amdgcn_readlane(my_phys, i);
        const int p = b0 + i;
        const int64_t meta = mb + p;
        if (phys < 0 || meta < 0 || meta > last_meta) return;
        const int valid = min(P, n - p * P);
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lo[e] = __builtin_inff();
          hi[e] = -__builtin_inff();
        }
#pragma unroll
        for (int k = 0; k < TL; ++k) {
          if (rg + RPL * k < valid) {
            const uint32_t w[4] = {src[k].x, src[k].y, src[k].z, src[k].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float a = lo_f(w[e], DT()), b = hi_f(w[e], DT());
              lo[2 * e] = fminf(lo[2 * e], a);
              hi[2 * e] = fmaxf(hi[2 * e], a);
              lo[2 * e + 1] = fminf(lo[2 * e + 1], b);
              hi[2 * e + 1] = fmaxf(hi[2 * e + 1], b);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lo[e] = -across_max<COLS>(-lo[e]);
          hi[e] = across_max<COLS>(hi[e]);
        }
        if (rg == 0) {
          uint16_t* mm = reinterpret_cast<uint16_t*>(c.minmax) + meta * 2 * D;
          uint4 a, b;
          a.x = pack2(lo[0], hi[0], DT());
          a.y = pack2(lo[1], hi[1], DT());
          a.z = pack2(lo[2], hi[2], DT());
          a.w = pack2(lo[3], hi[3], DT());
          b.x = pack2(lo[4], hi[4], DT());
          b.y = pack2(lo[5], hi[5], DT());
          b.z = pack2(lo[6], hi[6], DT());
          b.w = pack2(lo[7], hi[7], DT());
          *reinterpret_cast<uint4*>(mm + 16 * col) = a;
          *reinterpret_cast<uint4*>(mm + 16 * col + 8) = b;
        }
      };
      uint4 buf0[TL], buf1[TL];
      load(tile(0), buf0);
      for (int i = 0; i < nb; i += 2) {
        load(tile(min(i + 1, nb - 1)), buf1);
        reduce_store(i, buf0);
        load(tile(min(i + 2, nb - 1)), buf0);
        if (i + 1 < nb) reduce_store(i + 1, buf1);
      }
    }
    t0 = seg_end;
    while (hh < BH && uni(pre[hh + 1]) <= t0) ++hh;
  }
}

template <int D, typename DT>
const void* minmax_symbol() {
  return reinterpret_cast<const void*>(&minmax_kernel<D, DT>);
}

template <int D, typename DT>
hipError_t launch_d(const CacheView& c, hipStream_t s) {
  int grid = 0;
  if (hipError_t e = resident_grid<minmax_symbol<D, DT>>(&grid)) return e;
  const size_t lds = (size_t)(c.b * c.Hkv + 1) * sizeof(int);
  hipLaunchKernelGGL((minmax_kernel<D, DT>), dim3((unsigned)grid), dim3(kFlatThreads), lds, s, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_minmax(const CacheView& c, hipStream_t s) {
  if (c.dtype == KVS_F16) return c.d == 128 ? launch_d<128, F16>(c, s) : launch_d<256, F16>(c, s);
  return c.d == 128 ? launch_d<128, BF16>(c, s) : launch_d<256, BF16>(c, s);
}

}  // namespace kvs
