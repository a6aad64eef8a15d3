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
// then across the RPL row groups with lane swaps, taken on 16-bit order
// keys rather than floats: flipping the sign bit of a non-negative value
// and every bit of a negative one makes unsigned order equal float order,
// so packed u16 min/max treat two channels per instruction with no
// conversion, and the inverse map gives back the exact bits (-0 orders just
// below +0; both are the same value).  The output is
// channel-interleaved, (min, max) per channel, so that one page of one head
// is a single contiguous 4*d-byte block, and goes to block meta_base[r][h] +
// p of the min-max cache, not to the page's physical KV slot: each head's
// bounds form one contiguous run in page order.  K tiles are read with
// non-temporal loads (each once per build), never past a batch's last page;
// a missing page reads page 0 and is discarded.
#include "flat_pages.h"
#include "kvs_launch.h"

namespace kvs {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// Order keys of two fp16 / bf16 values, and their inverse.
__device__ __forceinline__ uint32_t to_keys(uint32_t w) {
  const uint32_t neg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, w) >> (short)15);
  return w ^ (neg | 0x80008000u);
}
__device__ __forceinline__ uint32_t from_keys(uint32_t k) {
  const uint32_t neg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, ~k) >> (short)15);
  return k ^ ((neg & 0x7fff7fffu) | 0x80008000u);
}
__device__ __forceinline__ uint32_t kmin(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t kmax(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
// min / max of packed keys across lanes that differ in lane bits >= FROM
// (FROM = 16 or 32)
template <int FROM>
__device__ __forceinline__ void across_keys(uint32_t& lo, uint32_t& hi) {
  if (FROM == 16) {
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    lo = kmin(l[0], l[1]);
    hi = kmax(h[0], h[1]);
  }
  const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  lo = kmin(l[0], l[1]);
  hi = kmax(h[0], h[1]);
}

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
        for (int k = 0; k < TL; ++k) dst[k] = ld16_once(t + RPL * k * D);
      };
      auto reduce_store = [&](int i, const uint4 (&src)[TL]) {
        const int phys = __builtin_amdgcn_readlane(my_phys, i);
        const int p = b0 + i;
        const int64_t meta = mb + p;
        if (phys < 0 || meta < 0 || meta > last_meta) return;
        const int valid = min(P, n - p * P);
        uint32_t lo[4], hi[4];   // keys of channels (2e, 2e + 1) of the lane's 8
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = 0xffffffffu;
          hi[e] = 0u;
        }
        auto row = [&](const uint4& v) {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = to_keys(w[e]);
            lo[e] = kmin(lo[e], key);
            hi[e] = kmax(hi[e], key);
          }
        };
        if (valid == P) {   // a full page (all but a head's last): no row masks
#pragma unroll
          for (int k = 0; k < TL; ++k) row(src[k]);
        } else {
#pragma unroll
          for (int k = 0; k < TL; ++k)
            if (rg + RPL * k < valid) row(src[k]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) across_keys<COLS>(lo[e], hi[e]);
        if (rg == 0) {
          // (min, max) of channel 2e from the low halves, of 2e + 1 from the high
          uint32_t o[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lb = from_keys(lo[e]), hb = from_keys(hi[e]);
            o[2 * e] = __builtin_amdgcn_perm(hb, lb, 0x05040100u);
            o[2 * e + 1] = __builtin_amdgcn_perm(hb, lb, 0x07060302u);
          }
          uint16_t* mm = reinterpret_cast<uint16_t*>(c.minmax) + meta * 2 * D;
          *reinterpret_cast<uint4*>(mm + 16 * col) = make_uint4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<uint4*>(mm + 16 * col + 8) = make_uint4(o[4], o[5], o[6], o[7]);
        }
      };
      uint4 buf0[TL], buf1[TL];
      load(tile(0), buf0);
      for (int i = 0; i < nb; i += 2) {   // no load past the batch (uniform tests)
        if (i + 1 < nb) load(tile(i + 1), buf1);
        reduce_store(i, buf0);
        if (i + 2 < nb) load(tile(i + 2), buf0);
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
