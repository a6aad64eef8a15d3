// Page scores and per-KV-head top-K in one launch (FlexiCache summary, Core
// method: Quest bounds rank a head's pages and the head attends only its K
// best).  One 256-thread workgroup per (request, KV head): its four waves
// score quarters of the head's pages with score_run (the same lanes,
// operations and order as the scoring kernel, so the scores are the same
// bits), writing order keys to LDS and, when asked, the scores to memory;
// after one barrier the block selection of radix_select.h takes the
// min(K, np) largest keys from LDS and writes the kept pages in ascending
// order, -1 past them.  The scores never make a round trip through memory
// and the selection needs no launch of its own; the price is one workgroup
// per head, which keeps the chip busy only when heads are many and of
// similar length (the workgroups of a short head idle while a long one is
// still streaming).
#include "kvs_launch.h"
#include "quest_bound.h"
#include "radix_select.h"

namespace kvs {
namespace {

constexpr int P = 16;
// Rounds of bounds per wave: one scored, one in flight (deeper rings measured
// slower here).
constexpr int kRing = 2;

constexpr int kRoundRegs = 32;   // 64 and 128 measured slower

#ifdef KVS_WG_STAMPS
// Instrumented build only: per workgroup of the last launch, the clock
// (s_memrealtime, 100 MHz) at entry [0], when wave w has scored its pages
// [1 + w], past the barrier after scoring [9], once the K-th key is known
// [10], and at exit [11], each stored when taken.
constexpr int kSelectStampBlocks = 16384;
constexpr int kSelectStamps = 12;
__device__ uint64_t g_select_stamps[kSelectStampBlocks][kSelectStamps];
#define KVS_SELECT_STAMP(k)                                                         \
  do {                                                                              \
    if (blockIdx.x < kSelectStampBlocks)                                            \
      g_select_stamps[blockIdx.x][k] = __builtin_amdgcn_s_memrealtime();            \
  } while (0)
#else
#define KVS_SELECT_STAMP(k) \
  do {                      \
  } while (0)
#endif

template <int D, int GQ, typename DT>
__global__ __launch_bounds__(kSelThreads) void select_pages_kernel(
    CacheView c, const uint16_t* __restrict__ q, float* __restrict__ scores, int K,
    int32_t* __restrict__ sel, int32_t* __restrict__ sel_count) {
  extern __shared__ uint32_t keys[];   // [maxpg]
  __shared__ SelectShared sh;
  const int rh = blockIdx.x;
  const int r = rh / c.Hkv, h = rh - r * c.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int ql = lane % 8;
  if (tid == 0) KVS_SELECT_STAMP(0);
  const int npg = (clampi(c.seq_len[rh], 0, P * c.maxpg) + P - 1) / P;
  const int keep = min(K, npg);
  const int hs = c.head_slot[h];
  const bool head_ok = hs >= 0 && hs < c.Hkv;
  const int gi = head_ok ? hs / c.Hp : 0;
  const int32_t* ptrow = c.page_table + ((int64_t)r * c.G + gi) * c.maxpg;
  const int64_t mb = c.meta_base[rh], last = c.num_meta - 1;
  const uint16_t* mmb = reinterpret_cast<const uint16_t*>(c.minmax) + 8 * ql;
  float* srow = scores ? scores + (int64_t)rh * c.maxpg : nullptr;

  const int p0 = (int)((int64_t)npg * wid / kSelWaves);
  const int p1 = (int)((int64_t)npg * (wid + 1) / kSelWaves);
  if (p0 < p1) {
    QuestQuery<D, GQ> qq;
    qq.load(q + ((int64_t)r * c.Hq + h * GQ) * D, ql);
    score_run<D, GQ, DT, kRing, kRoundRegs>(qq, mmb, mb, last, ptrow, c.num_pages, head_ok, p0, p1, lane,
                         [&](int p, float v) {
                           keys[p] = order_key(v);
                           if (srow) srow[p] = v;
                         });
  }
  if (srow)
    for (int p = npg + tid; p < c.maxpg; p += kSelThreads) srow[p] = -__builtin_inff();
  if (lane == 0) KVS_SELECT_STAMP(1 + wid);
  __syncthreads();
  if (tid == 0) KVS_SELECT_STAMP(9);

  int32_t* out = sel + (int64_t)rh * K;
  const Threshold th = kth_largest(keys, npg, keep, sh);
  if (tid == 0) KVS_SELECT_STAMP(10);
  place_kept(keys, npg, keep, th, sh, [&](int pos, int p) { out[pos] = p; });
  for (int k = keep + tid; k < K; k += kSelThreads) out[k] = -1;
  if (tid == 0) sel_count[rh] = keep;
  if (tid == 0) KVS_SELECT_STAMP(11);
}

template <int D, int GQ, typename DT>
hipError_t launch_v(const CacheView& c, const void* q, float* scores, int K, int32_t* sel,
                    int32_t* sel_count, hipStream_t s) {
  const size_t lds = (size_t)c.maxpg * sizeof(uint32_t);
  hipLaunchKernelGGL((select_pages_kernel<D, GQ, DT>), dim3((unsigned)(c.b * c.Hkv)),
                     dim3(kSelThreads), lds, s, c, static_cast<const uint16_t*>(q), scores, K, sel,
                     sel_count);
  return hipGetLastError();
}

template <int D, typename DT>
hipError_t launch_g(const CacheView& c, const void* q, float* scores, int K, int32_t* sel,
                    int32_t* sel_count, hipStream_t s) {
  switch (c.Gq) {
    case 1: return launch_v<D, 1, DT>(c, q, scores, K, sel, sel_count, s);
    case 2: return launch_v<D, 2, DT>(c, q, scores, K, sel, sel_count, s);
    case 4: return launch_v<D, 4, DT>(c, q, scores, K, sel, sel_count, s);
    default: return launch_v<D, 8, DT>(c, q, scores, K, sel, sel_count, s);
  }
}

}  // namespace

#ifdef KVS_WG_STAMPS
hipError_t copy_select_stamps(uint64_t* dst, size_t blocks, hipStream_t s) {
  void* src = nullptr;
  if (hipError_t e = hipGetSymbolAddress(&src, HIP_SYMBOL(g_select_stamps))) return e;
  if (blocks > (size_t)kSelectStampBlocks) blocks = kSelectStampBlocks;
  return hipMemcpyAsync(dst, src, blocks * kSelectStamps * sizeof(uint64_t),
                        hipMemcpyDeviceToDevice, s);
}
#endif

hipError_t launch_select(const CacheView& c, const void* q, float* scores, int K, int32_t* sel,
                         int32_t* sel_count, hipStream_t s) {
  if (c.dtype == KVS_F16)
    return c.d == 128 ? launch_g<128, F16>(c, q, scores, K, sel, sel_count, s)
                      : launch_g<256, F16>(c, q, scores, K, sel, sel_count, s);
  return c.d == 128 ? launch_g<128, BF16>(c, q, scores, K, sel, sel_count, s)
                    : launch_g<256, BF16>(c, q, scores, K, sel, sel_count, s);
}

}  // namespace kvs
