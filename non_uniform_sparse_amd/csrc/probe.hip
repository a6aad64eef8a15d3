// Read-only probe of the decode's gather: the K and V tiles of every
// attended (request, head, page) unit, found through the page table exactly
// as the decode finds them, read from HBM with no arithmetic beyond folding
// the loaded words into one value per wave (so no load can be dropped).
// Its rate is the empirical ceiling of the decode's access pattern on the
// chip; the decode's own rate is set against it.
//
// The grid is resident-sized and each wave takes an even share of all heads'
// units (flat_pages.h).  A unit's K tile and V tile are 2 P d contiguous
// elements; 64 lanes read 16 bytes each per load instruction, and the next
// unit's loads are issued before the current one is folded; no load reaches
// past a segment's last unit.  A missing (null) page loads page 0's tile,
// and those words are not folded.
#include "flat_pages.h"
#include "kvs_launch.h"

namespace kvs {
namespace {

__device__ __forceinline__ int unit_count(const CacheView& c, const int32_t* sel_count, int K,
                                          int rh) {
  constexpr int P = 16;
  const int npg = (clampi(c.seq_len[rh], 0, P * c.maxpg) + P - 1) / P;
  return sel_count ? clampi(sel_count[rh], 0, min(K, npg)) : npg;
}

template <int D>
__global__ __launch_bounds__(kFlatThreads) void probe_kernel(CacheView c, const int32_t* sel,
                                                             const int32_t* sel_count, int K,
                                                             uint32_t* sink) {
  constexpr int P = 16;
  constexpr int LOADS = 2 * P * D * 2 / (64 * 16);   // 16-byte loads per lane per unit
  extern __shared__ int pre[];
  __shared__ int part[kFlatThreads];
  const int BH = c.b * c.Hkv;
  page_prefix(BH, [&](int rh) { return unit_count(c, sel_count, K, rh); }, pre, part);
  const int lane = threadIdx.x & 63;
  const FlatShare share = flat_share(pre, BH);
  int t0 = share.t0, hh = share.hh;
  const int t1 = share.t1;
  const uint16_t* kvb = reinterpret_cast<const uint16_t*>(c.kv) + 8 * lane;
  uint32_t acc = 0;

  while (t0 < t1) {
    const int rh = hh;
    const int base = uni(pre[rh]);
    const int seg_end = min(t1, uni(pre[rh + 1]));
    const int i0 = t0 - base, i1 = seg_end - base;   // units [i0, i1) of head rh
    const int r = rh / c.Hkv, h = rh - r * c.Hkv;
    const int hs = c.head_slot[h];
    const bool head_ok = hs >= 0 && hs < c.Hkv;
    const int gi = head_ok ? hs / c.Hp : 0, slot = head_ok ? hs % c.Hp : 0;
    const int32_t* ptrow = c.page_table + ((int64_t)r * c.G + gi) * c.maxpg;
    const int32_t* srow = sel ? sel + (int64_t)rh * K : nullptr;
    // unit i's tile; ok = false for a null or out-of-range page
    auto tile = [&](int i, bool& ok) {
      int p = srow ? srow[i] : i;
      p = clampi(p, 0, c.maxpg - 1);
      const int phys = ptrow[p];
      ok = head_ok && phys >= 0 && phys < c.num_pages;
      return kvb + (ok ? ((int64_t)phys * c.Hp + slot) * 2 * P * D : 0);
    };
    uint4 buf0[LOADS], buf1[LOADS];
    bool ok0, ok1;
    auto load = [&](int i, uint4 (&dst)[LOADS], bool& ok) {
      const uint16_t* t = tile(i, ok);
#pragma unroll
      for (int k = 0; k < LOADS; ++k) dst[k] = ld16_once(t + 512 * k);
    };
    auto fold = [&](const uint4 (&src)[LOADS], bool ok) {
      uint32_t x = 0;
#pragma unroll
      for (int k = 0; k < LOADS; ++k) x ^= src[k].x ^ src[k].y ^ src[k].z ^ src[k].w;
      acc ^= ok ? x : 0u;
    };
    load(i0, buf0, ok0);
    for (int i = i0; i < i1; i += 2) {   // no load past the segment (uniform tests)
      if (i + 1 < i1) load(i + 1, buf1, ok1);
      fold(buf0, ok0);
      if (i + 2 < i1) load(i + 2, buf0, ok0);
      if (i + 1 < i1) fold(buf1, ok1);
    }
    t0 = seg_end;
    while (hh < BH && uni(pre[hh + 1]) <= t0) ++hh;
  }
  // one word per wave: the fold of all its lanes
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (lane == 0) sink[(int64_t)blockIdx.x * (kFlatThreads / 64) + (threadIdx.x >> 6)] = acc;
}

template <int D>
const void* probe_symbol() {
  return reinterpret_cast<const void*>(&probe_kernel<D>);
}

template <int D>
hipError_t launch_d(const CacheView& c, const int32_t* sel, const int32_t* sel_count, int K,
                    uint32_t* sink, size_t sink_words, hipStream_t s) {
  int grid = 0;
  if (hipError_t e = resident_grid<probe_symbol<D>>(&grid)) return e;
  if ((size_t)grid * (kFlatThreads / 64) > sink_words) return hipErrorInvalidValue;
  const size_t lds = (size_t)(c.b * c.Hkv + 1) * sizeof(int);
  hipLaunchKernelGGL((probe_kernel<D>), dim3((unsigned)grid), dim3(kFlatThreads), lds, s, c, sel,
                     sel_count, K, sink);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_probe(const CacheView& c, const int32_t* sel, const int32_t* sel_count, int K,
                        uint32_t* sink, size_t sink_words, hipStream_t s) {
  return c.d == 128 ? launch_d<128>(c, sel, sel_count, K, sink, sink_words, s)
                    : launch_d<256>(c, sel, sel_count, K, sink, sink_words, s);
}

int probe_sink_words(int d, int* words) {
  int grid = 0;
  const hipError_t e = d == 128 ? resident_grid<probe_symbol<128>>(&grid)
                                : resident_grid<probe_symbol<256>>(&grid);
  if (e) return -1;
  *words = grid * (kFlatThreads / 64);
  return 0;
}

}  // namespace kvs
