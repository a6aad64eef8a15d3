// One chunk of a chunked prefill under Budget Reservation (Tangram review,
// 3.1: as each chunk's K/V is computed every head keeps its top tokens by a
// score, so the compressed footprint is fixed when the request is scheduled;
// 3.2 Ragged Paging: kept tokens go into the head's slot of its group's
// pages; FlexiCache summary, Key observations, assumption 2: the pages'
// min-max bounds are kept current on the GPU).
//
// Two kernels.  select_kernel, one 256-thread workgroup per (request, KV
// head): the chunk's C scores become keys in LDS and the block selection of
// radix_select.h keeps the quota largest (equal scores to the lower
// position); the kept tokens' positions, in position order, the head's
// length before the chunk and the quota go to the workspace, and the length
// advances.  place_kernel, one wave per page the chunk writes into (a grid
// over (head, page)): kept token j lands in row (n + j) % P of page
// (n + j) / P; lane l moves 16 bytes of K and of V of rows rg + RPL*k
// (rg = l / COLS), so each load covers RPL whole rows, stores them into the
// page and reduces the K pieces into the page's per-channel bounds (lane
// swaps across the RPL row groups), merging with the bounds the page held
// when it already had tokens before this chunk.  Every row's K and V is
// read once and written once.
#include "radix_select.h"
#include "kvs_launch.h"

namespace kvs {
namespace {

constexpr int P = 16;
constexpr int kPagesPerBlock = 4;   // one page per wave

// Per-head workspace record: length before the chunk, quota, kept positions.
struct HeadChunk {
  int n, q;
};

__host__ __device__ inline int64_t head_record_bytes(int C) {
  return ((int64_t)sizeof(HeadChunk) + (int64_t)C * sizeof(uint16_t) + 15) / 16 * 16;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(CacheView c,
                                                             const float* __restrict__ scores,
                                                             const int32_t* __restrict__ quota,
                                                             int C, uint8_t* __restrict__ ws) {
  extern __shared__ uint32_t keys[];   // [C]
  __shared__ SelectShared sh;
  const int rh = blockIdx.x;
  const int h = rh % c.Hkv;
  const int tid = threadIdx.x;
  const int n = clampi(c.seq_len[rh], 0, P * c.maxpg);
  const int hs = c.head_slot[h];
  // a head with an invalid slot keeps nothing (and its length stays)
  const int q = (hs < 0 || hs >= c.Hkv) ? 0 : clampi(quota[rh], 0, min(C, P * c.maxpg - n));
  uint8_t* rec = ws + rh * head_record_bytes(C);
  uint16_t* kept = reinterpret_cast<uint16_t*>(rec + sizeof(HeadChunk));

  load_keys(scores + (int64_t)rh * C, C, keys);
  const Threshold th = kth_largest(keys, C, q, sh);
  place_kept(keys, C, q, th, sh, [&](int pos, int t) { kept[pos] = (uint16_t)t; });
  if (tid == 0) {
    *reinterpret_cast<HeadChunk*>(rec) = HeadChunk{n, q};
    c.seq_len[rh] = n + q;
  }
}

template <int D, typename DT>
__global__ __launch_bounds__(64 * kPagesPerBlock) void place_kernel(
    CacheView c, const uint16_t* __restrict__ k_chunk, const uint16_t* __restrict__ v_chunk, int C,
    const uint8_t* __restrict__ ws) {
  constexpr int COLS = D / 8;      // lanes per row
  constexpr int RPL = 64 / COLS;   // rows per load
  constexpr int TL = P / RPL;      // rows per lane
  const int rh = blockIdx.y;
  const int r = rh / c.Hkv, h = rh % c.Hkv;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kPagesPerBlock + (threadIdx.x >> 6);   // touched page of the head
  const uint8_t* rec = ws + rh * head_record_bytes(C);
  const HeadChunk hc = *reinterpret_cast<const HeadChunk*>(rec);
  const uint16_t* kept = reinterpret_cast<const uint16_t*>(rec + sizeof(HeadChunk));
  const int n = hc.n, q = hc.q;
  if (q <= 0) return;
  const int p = n / P + i;
  if (p > (n + q - 1) / P) return;
  const int hs = c.head_slot[h];
  const int gi = hs / c.Hp, slot = hs % c.Hp;   // q > 0 only for a valid slot
  const int phys = c.page_table[((int64_t)r * c.G + gi) * c.maxpg + p];
  const int64_t meta = (int64_t)c.meta_base[rh] + p;
  if (phys < 0 || phys >= c.num_pages) return;
  const int lo_pos = max(n, p * P), hi_pos = min(n + q, (p + 1) * P);

  const int rg = lane / COLS, col = lane % COLS;
  const uint16_t* ksrc = k_chunk + (int64_t)rh * C * D + 8 * col;
  const uint16_t* vsrc = v_chunk + (int64_t)rh * C * D + 8 * col;
  uint16_t* tile = reinterpret_cast<uint16_t*>(c.kv) + ((int64_t)phys * c.Hp + slot) * 2 * P * D + 8 * col;
  uint4 kr[TL], vr[TL];
#pragma unroll
  for (int k = 0; k < TL; ++k) {   // row rg + RPL k of the page, clamped into the chunk's rows
    const int pos = min(max(p * P + rg + RPL * k, lo_pos), hi_pos - 1);
    const int64_t t = kept[pos - n];
    kr[k] = ld16_once(ksrc + t * D);
    vr[k] = ld16_once(vsrc + t * D);
  }
  float lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = __builtin_inff();
    hi[e] = -__builtin_inff();
  }
#pragma unroll
  for (int k = 0; k < TL; ++k) {
    const int row = rg + RPL * k;
    const int pos = p * P + row;
    if (pos < lo_pos || pos >= hi_pos) continue;
    *reinterpret_cast<uint4*>(tile + row * D) = kr[k];
    *reinterpret_cast<uint4*>(tile + P * D + row * D) = vr[k];
    const uint32_t w[4] = {kr[k].x, kr[k].y, kr[k].z, kr[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = lo_f(w[e], DT()), b = hi_f(w[e], DT());
      lo[2 * e] = fminf(lo[2 * e], a);
      hi[2 * e] = fmaxf(hi[2 * e], a);
      lo[2 * e + 1] = fminf(lo[2 * e + 1], b);
      hi[2 * e + 1] = fmaxf(hi[2 * e + 1], b);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = -across_max<COLS>(-lo[e]);
    hi[e] = across_max<COLS>(hi[e]);
  }
  if (rg == 0 && meta >= 0 && meta < c.num_meta) {
    uint16_t* mm = reinterpret_cast<uint16_t*>(c.minmax) + meta * 2 * D + 16 * col;
    if (p * P < n) {   // the page held tokens before this chunk: merge
      const uint4 a = ld16(mm), b = ld16(mm + 8);
      const uint32_t ow[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        lo[ch] = fminf(lo[ch], lo_f(ow[ch], DT()));
        hi[ch] = fmaxf(hi[ch], hi_f(ow[ch], DT()));
      }
    }
    uint4 a, b;
    a.x = pack2(lo[0], hi[0], DT());
    a.y = pack2(lo[1], hi[1], DT());
    a.z = pack2(lo[2], hi[2], DT());
    a.w = pack2(lo[3], hi[3], DT());
    b.x = pack2(lo[4], hi[4], DT());
    b.y = pack2(lo[5], hi[5], DT());
    b.z = pack2(lo[6], hi[6], DT());
    b.w = pack2(lo[7], hi[7], DT());
    *reinterpret_cast<uint4*>(mm) = a;
    *reinterpret_cast<uint4*>(mm + 8) = b;
  }
}

template <int D, typename DT>
hipError_t launch_d(const CacheView& c, const void* k_chunk, const void* v_chunk,
                    const float* scores, const int32_t* quota, int C, void* ws, hipStream_t s) {
  const int BH = c.b * c.Hkv;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)BH), dim3(kSelThreads),
                     (size_t)C * sizeof(uint32_t), s, c, scores, quota, C,
                     static_cast<uint8_t*>(ws));
  if (hipError_t e = hipGetLastError()) return e;
  const int pages = C / P + 2;   // pages one chunk can write into
  const dim3 grid((unsigned)((pages + kPagesPerBlock - 1) / kPagesPerBlock), (unsigned)BH);
  hipLaunchKernelGGL((place_kernel<D, DT>), grid, dim3(64 * kPagesPerBlock), 0, s, c,
                     static_cast<const uint16_t*>(k_chunk), static_cast<const uint16_t*>(v_chunk),
                     C, static_cast<const uint8_t*>(ws));
  return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int b, int Hkv, int C) {
  return (size_t)b * Hkv * head_record_bytes(C);
}

hipError_t launch_prefill(const CacheView& c, const void* k_chunk, const void* v_chunk,
                          const float* scores, const int32_t* quota, int C, void* ws,
                          hipStream_t s) {
  if (c.dtype == KVS_F16)
    return c.d == 128 ? launch_d<128, F16>(c, k_chunk, v_chunk, scores, quota, C, ws, s)
                      : launch_d<256, F16>(c, k_chunk, v_chunk, scores, quota, C, ws, s);
  return c.d == 128 ? launch_d<128, BF16>(c, k_chunk, v_chunk, scores, quota, C, ws, s)
                    : launch_d<256, BF16>(c, k_chunk, v_chunk, scores, quota, C, ws, s);
}

}  // namespace kvs
