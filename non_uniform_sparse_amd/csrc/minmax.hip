// Min-max page metadata builder (FlexiCache summary, Key observations,
// assumption 2: per-page key bounds kept on the GPU, apart from the KV pages).
//
// One wave per (request, KV head, logical page).  A page's K tile is P = 16
// rows of d contiguous elements; lane l reads 16 bytes (8 channels) of row
// rg + RPL*k, rg = l / COLS, so each load instruction covers RPL whole rows
// (1 KB) and the tile is read once, fully coalesced.  Per-channel min/max
// over the lane's rows, then across the RPL row groups with lane swaps.  The
// output is channel-interleaved, (min, max) per channel, so that one page of
// one head is a single contiguous 4*d-byte block, and goes to block
// meta_base[r][h] + p of the min-max cache, not to the page's physical KV
// slot: each head's bounds form one contiguous run in page order.
#include "kvs_device.h"

namespace kvs {
namespace {

template <int D, typename DT>
__global__ __launch_bounds__(256) void minmax_kernel(CacheView c) {
  constexpr int P = 16;
  constexpr int COLS = D / 8;      // lanes per row
  constexpr int RPL = 64 / COLS;   // rows per load
  constexpr int TL = P / RPL;      // rows per lane
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = (int64_t)c.b * c.Hkv * c.maxpg;
  if (wave >= total) return;
  const int p = (int)(wave % c.maxpg);
  const int h = (int)((wave / c.maxpg) % c.Hkv);
  const int r = (int)(wave / ((int64_t)c.maxpg * c.Hkv));
  const int n = clampi(c.seq_len[r * c.Hkv + h], 0, P * c.maxpg);
  if (p * P >= n) return;
  const int hs = c.head_slot[h];
  if (hs < 0 || hs >= c.Hkv) return;
  const int gi = hs / c.Hp, slot = hs % c.Hp;
  const int phys = c.page_table[((int64_t)r * c.G + gi) * c.maxpg + p];
  if (phys < 0 || phys >= c.num_pages) return;
  const int64_t meta = (int64_t)c.meta_base[r * c.Hkv + h] + p;
  if (meta < 0 || meta >= c.num_meta) return;
  const int valid = min(P, n - p * P);

  const int rg = lane / COLS, col = lane % COLS;
  const uint16_t* ktile = reinterpret_cast<const uint16_t*>(c.kv) +
                          ((int64_t)phys * c.Hp + slot) * 2 * P * D;
  float lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = __builtin_inff();
    hi[e] = -__builtin_inff();
  }
#pragma unroll
  for (int k = 0; k < TL; ++k) {
    const int t = rg + RPL * k;
    if (t < valid) {
      const uint4 v = ld16(ktile + t * D + 8 * col);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
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
    // channel-interleaved: (min, max) of channel ch at elements 2 ch, 2 ch + 1
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
}

template <int D, typename DT>
hipError_t launch_d(const CacheView& c, hipStream_t s) {
  const int64_t waves = (int64_t)c.b * c.Hkv * c.maxpg;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((minmax_kernel<D, DT>), dim3((unsigned)blocks), dim3(256), 0, s, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_minmax(const CacheView& c, hipStream_t s) {
  if (c.dtype == KVS_F16) return c.d == 128 ? launch_d<128, F16>(c, s) : launch_d<256, F16>(c, s);
  return c.d == 128 ? launch_d<128, BF16>(c, s) : launch_d<256, BF16>(c, s);
}

}  // namespace kvs
