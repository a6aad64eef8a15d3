// Read-only probe of the decode's gather: the K and V tiles of every
// attended (request, head, page) unit, found through the page table exactly
// as the decode finds them, read from HBM with no arithmetic beyond folding
// the loaded words into one value per wave (so no load can be dropped).
// Its rate is the empirical ceiling of the decode's access pattern on the
// chip; the decode's own rate is set against it.
//
// The grid is resident-sized and each wave takes an even share of all heads'
// units (flat_pages.h).  As in the decode, a wave resolves the physical ids
// of 64 units at a time, lane-parallel (selection entry, then page table),
// and reads them back with readlane.  A unit's K tile and V tile are 2 P d
// contiguous elements; 64 lanes read 16 bytes each per load instruction
// (non-temporal), and the next unit's loads are issued before the current
// one is folded; no load reaches past a batch's last unit.  A missing (null)
// page loads page 0's tile, and those words are not folded.
//
// A second probe reads plain contiguous memory: the rate of a launch of a
// given size with no gather at all, for comparing a kernel with a stream of
// its own byte count.
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
    uint4 buf0[LOADS], buf1[LOADS];
    auto load = [&](const uint16_t* t, uint4 (&dst)[LOADS]) {
#pragma unroll
      for (int k = 0; k < LOADS; ++k) dst[k] = ld16_once(t + 512 * k);
    };
    auto fold = [&](const uint4 (&src)[LOADS], bool ok) {
      uint32_t x = 0;
#pragma unroll
      for (int k = 0; k < LOADS; ++k) x ^= src[k].x ^ src[k].y ^ src[k].z ^ src[k].w;
      acc ^= ok ? x : 0u;
    };
    for (int b0 = i0; b0 < i1; b0 += 64) {
      const int nb = min(64, i1 - b0);
      // lane u resolves unit b0 + u (selection entry, then page table), as
      // the decode does; -1: null or out-of-range page
      int my_phys = -1;
      if (lane < nb) {
        int p = srow ? srow[b0 + lane] : b0 + lane;
        p = clampi(p, 0, c.maxpg - 1);
        const int ph = ptrow[p];
        if (head_ok && ph >= 0 && ph < c.num_pages) my_phys = ph;
      }
      auto phys_of = [&](int u) { return __builtin_amdgcn_readlane(my_phys, u); };
      auto tile = [&](int u) {
        const int ph = phys_of(u);
        return kvb + (ph >= 0 ? ((int64_t)ph * c.Hp + slot) * 2 * P * D : 0);
      };
      load(tile(0), buf0);
      for (int u = 0; u < nb; u += 2) {   // no load past the batch (uniform tests)
        if (u + 1 < nb) load(tile(u + 1), buf1);
        fold(buf0, phys_of(u) >= 0);
        if (u + 2 < nb) load(tile(u + 2), buf0);
        if (u + 1 < nb) fold(buf1, phys_of(u + 1) >= 0);
      }
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

// Plain read of n16 16-byte words: wave w of W reads words [n16 w/W,
// n16 (w+1)/W), 64 lanes x CH non-temporal loads per step (CH KB per step),
// two steps in flight, and folds them into one sink word.
__global__ __launch_bounds__(kFlatThreads) void stream_probe_kernel(const uint4* __restrict__ src,
                                                                    int64_t n16,
                                                                    uint32_t* __restrict__ sink) {
  constexpr int CH = 8;
  const int lane = threadIdx.x & 63;
  const int64_t W = (int64_t)gridDim.x * (kFlatThreads / 64);
  const int64_t w = (int64_t)blockIdx.x * (kFlatThreads / 64) + (threadIdx.x >> 6);
  const int64_t lo = n16 * w / W, hi = n16 * (w + 1) / W;
  uint32_t acc = 0;
  uint4 b0[CH], b1[CH];
  auto load = [&](int64_t base, uint4 (&dst)[CH]) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int64_t i = base + 64 * k + lane;
      dst[k] = i < hi ? ld16_once(src + i) : make_uint4(0, 0, 0, 0);
    }
  };
  auto fold = [&](const uint4 (&v)[CH]) {
#pragma unroll
    for (int k = 0; k < CH; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  };
  constexpr int64_t STEP = 64 * CH;
  if (lo < hi) load(lo, b0);
  for (int64_t base = lo; base < hi; base += 2 * STEP) {   // no load past hi (uniform tests)
    if (base + STEP < hi) load(base + STEP, b1);
    fold(b0);
    if (base + 2 * STEP < hi) load(base + 2 * STEP, b0);
    if (base + STEP < hi) fold(b1);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (lane == 0) sink[w] = acc;
}

const void* stream_probe_symbol() { return reinterpret_cast<const void*>(&stream_probe_kernel); }

}  // namespace

hipError_t launch_stream_probe(const void* src, size_t bytes, uint32_t* sink, size_t sink_words,
                               hipStream_t s) {
  int grid = 0;
  if (hipError_t e = resident_grid<stream_probe_symbol>(&grid)) return e;
  if ((size_t)grid * (kFlatThreads / 64) > sink_words) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_probe_kernel, dim3((unsigned)grid), dim3(kFlatThreads), 0, s,
                     static_cast<const uint4*>(src), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

int stream_probe_sink_words(int* words) {
  int grid = 0;
  if (resident_grid<stream_probe_symbol>(&grid)) return -1;
  *words = grid * (kFlatThreads / 64);
  return 0;
}

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
