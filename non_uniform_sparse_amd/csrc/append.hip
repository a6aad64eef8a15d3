// Append of the decoded token (FlexiCache summary, Method: the token being
// decoded joins the cache before the step attends it; Key observations,
// assumption 2: the min-max bounds of its page are kept current on the GPU,
// so the page can be scored at any later step; Tangram review, 3.2 Ragged
// Paging: the token goes into its head's slot of the group's page).
//
// With a host tier (FlexiCache summary, tiered placement: the pages of a
// stable head live in host memory, newly filled ones included), a tiered
// head's row is written through to its host page host_base + n / P, and to
// its GPU copy too when that page is resident; the host copy stays complete,
// so a later promotion brings the new tokens along.
//
// One wave per (request, KV head).  With n = seq_len, the token lands in row
// n % P of logical page n / P.  Lanes [0, d/8) carry 8 channels of K each:
// they store the K row and merge the channels into the page's
// channel-interleaved (min, max) block, starting fresh when the row is the
// page's first; lanes [d/8, d/4) store the V row.  Lane 0 then advances n.
// Every skip condition is uniform over the wave.
#include "kvs_device.h"
#include "kvs_launch.h"

namespace kvs {
namespace {

template <int D, typename DT>
__global__ __launch_bounds__(256) void append_kernel(CacheView c, HostTierView t,
                                                     const uint16_t* __restrict__ k_new,
                                                     const uint16_t* __restrict__ v_new) {
  constexpr int P = 16;
  constexpr int LPR = D / 8;   // lanes per 16-bit row of d channels
  const int lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= (int64_t)c.b * c.Hkv) return;
  const int r = (int)(rh / c.Hkv), h = (int)(rh % c.Hkv);
  const int n = c.seq_len[rh];
  if (n < 0 || n >= P * c.maxpg) return;
  const int hs = c.head_slot[h];
  if (hs < 0 || hs >= c.Hkv) return;
  const int gi = hs / c.Hp, slot = hs % c.Hp;
  const int p = n / P, row = n % P;
  const int phys = c.page_table[((int64_t)r * c.G + gi) * c.maxpg + p];
  const bool resident = phys >= 0 && phys < c.num_pages;
  const int64_t hb = t.host_kv ? t.host_base[rh] : -1;
  const bool tiered = hb >= 0 && hb + p < t.num_host_pages;
  if (!resident && !tiered) return;
  const int64_t meta = (int64_t)c.meta_base[rh] + p;
  if (meta < 0 || meta >= c.num_meta) return;

  uint16_t* tile = resident ? reinterpret_cast<uint16_t*>(c.kv) + ((int64_t)phys * c.Hp + slot) * 2 * P * D
                            : nullptr;
  uint16_t* host = tiered ? static_cast<uint16_t*>(t.host_kv) + (hb + p) * 2 * P * D : nullptr;
  if (lane < LPR) {
    const uint4 k = ld16(k_new + rh * D + 8 * lane);
    if (resident) *reinterpret_cast<uint4*>(tile + row * D + 8 * lane) = k;
    if (tiered) *reinterpret_cast<uint4*>(host + row * D + 8 * lane) = k;
    uint16_t* mm = reinterpret_cast<uint16_t*>(c.minmax) + meta * 2 * D + 16 * lane;
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
    float lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[2 * e] = hi[2 * e] = lo_f(kw[e], DT());
      lo[2 * e + 1] = hi[2 * e + 1] = hi_f(kw[e], DT());
    }
    if (row > 0) {   // merge with the bounds of the rows already in the page
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
  } else if (lane < 2 * LPR) {
    const int l = lane - LPR;
    const uint4 v = ld16(v_new + rh * D + 8 * l);
    if (resident) *reinterpret_cast<uint4*>(tile + P * D + row * D + 8 * l) = v;
    if (tiered) *reinterpret_cast<uint4*>(host + P * D + row * D + 8 * l) = v;
  }
  if (lane == 0) c.seq_len[rh] = n + 1;
}

template <int D, typename DT>
hipError_t launch_d(const CacheView& c, const HostTierView& t, const void* k_new, const void* v_new,
                    hipStream_t s) {
  const int64_t waves = (int64_t)c.b * c.Hkv;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((append_kernel<D, DT>), dim3((unsigned)blocks), dim3(256), 0, s, c, t,
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const CacheView& c, const HostTierView* tier, const void* k_new,
                         const void* v_new, hipStream_t s) {
  HostTierView t{};
  if (tier) t = *tier;   // host_kv == nullptr: no host tier
  if (c.dtype == KVS_F16)
    return c.d == 128 ? launch_d<128, F16>(c, t, k_new, v_new, s) : launch_d<256, F16>(c, t, k_new, v_new, s);
  return c.d == 128 ? launch_d<128, BF16>(c, t, k_new, v_new, s) : launch_d<256, BF16>(c, t, k_new, v_new, s);
}

}  // namespace kvs
