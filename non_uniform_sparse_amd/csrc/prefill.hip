// One chunk of a chunked prefill under Budget Reservation (Tangram review,
// 3.1: as each chunk's K/V is computed every head keeps its top tokens by a
// score, so the compressed footprint is fixed when the request is scheduled;
// 3.2 Ragged Paging: kept tokens go into the head's slot of its group's
// pages; FlexiCache summary, Key observations, assumption 2: the pages'
// min-max bounds are kept current on the GPU).
//
// One 256-thread workgroup per (request, KV head).  The chunk's C scores
// become keys in LDS and the block selection of radix_select.h keeps the
// quota largest (equal scores to the lower position), listing the kept
// tokens in position order in LDS, next to the physical ids of the pages
// they land in.  The copy is flat over 16-byte pieces of the kept K and V
// rows, consecutive threads on consecutive pieces of a row, 16 loads in
// flight per thread before their stores: kept token j goes to row
// (n + j) % P of page (n + j) / P.  Then each wave rebuilds the bounds of
// one touched page at a time from the source rows of the tokens it received
// (all of a lane's rows loaded at once; RPL row groups merged by lane
// swaps), merging with the page's existing bounds when the page already
// held tokens before this chunk.  Finally n advances by the quota.
#include "radix_select.h"

namespace kvs {
namespace {

template <int D, typename DT>
__global__ __launch_bounds__(kSelThreads) void prefill_kernel(CacheView c,
                                                              const uint16_t* __restrict__ k_chunk,
                                                              const uint16_t* __restrict__ v_chunk,
                                                              const float* __restrict__ scores,
                                                              const int32_t* __restrict__ quota,
                                                              int C) {
  constexpr int P = 16;
  constexpr int COLS = D / 8;      // lanes per row
  constexpr int RPL = 64 / COLS;   // rows per load
  constexpr int TL = P / RPL;      // rows per lane of a page
  // LDS: keys[C], page ids [C / P + 2], kept[C] (16-bit: C <= 8192)
  extern __shared__ uint32_t lds[];
  uint32_t* keys = lds;
  int* pg = reinterpret_cast<int*>(lds + C);
  uint16_t* kept = reinterpret_cast<uint16_t*>(pg + C / P + 2);
  __shared__ SelectShared sh;
  const int rh = blockIdx.x;
  const int r = rh / c.Hkv, h = rh % c.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = clampi(c.seq_len[rh], 0, P * c.maxpg);
  const int q = clampi(quota[rh], 0, min(C, P * c.maxpg - n));
  const int hs = c.head_slot[h];
  if (hs < 0 || hs >= c.Hkv) return;   // the whole block: nothing written, n unchanged
  const int gi = hs / c.Hp, slot = hs % c.Hp;
  const int32_t* ptrow = c.page_table + ((int64_t)r * c.G + gi) * c.maxpg;
  const uint16_t* ksrc = k_chunk + (int64_t)rh * C * D;
  const uint16_t* vsrc = v_chunk + (int64_t)rh * C * D;
  uint16_t* pool = reinterpret_cast<uint16_t*>(c.kv);

  load_keys(scores + (int64_t)rh * C, C, keys);
  const Threshold th = kth_largest(keys, C, q, sh);
  place_kept(keys, C, q, th, sh, [&](int pos, int t) { kept[pos] = (uint16_t)t; });
  const int p_first = n / P;
  const int touched = q > 0 ? (n + q - 1) / P - p_first + 1 : 0;   // <= C / P + 2
  for (int i = tid; i < touched; i += kSelThreads) {
    const int phys = ptrow[p_first + i];
    pg[i] = phys >= 0 && phys < c.num_pages ? phys : -1;
  }
  __syncthreads();

  // copy: 16-byte pieces of the kept K and V rows, flat over the block
  constexpr int IT = 16;
  const int items = q * 2 * COLS;
  for (int base = 0; base < items; base += kSelThreads * IT) {
    uint4 v[IT];
#pragma unroll
    for (int u = 0; u < IT; ++u) {
      const int item = min(base + u * kSelThreads + tid, items - 1);
      const int j = item / (2 * COLS), rem = item % (2 * COLS);
      const uint16_t* src = (rem < COLS ? ksrc : vsrc) + (int64_t)kept[j] * D + 8 * (rem % COLS);
      v[u] = ld16(src);
    }
#pragma unroll
    for (int u = 0; u < IT; ++u) {
      const int item = base + u * kSelThreads + tid;
      if (item < items) {
        const int j = item / (2 * COLS), rem = item % (2 * COLS);
        const int pos = n + j;
        const int phys = pg[pos / P - p_first];
        if (phys >= 0) {
          uint16_t* dst = pool + ((int64_t)phys * c.Hp + slot) * 2 * P * D +
                          (rem < COLS ? 0 : P * D) + (pos % P) * D + 8 * (rem % COLS);
          *reinterpret_cast<uint4*>(dst) = v[u];
        }
      }
    }
  }

  // bounds of every page the chunk wrote into, one page per wave at a time
  if (q > 0) {
    const int rg = lane / COLS, col = lane % COLS;
    const int64_t mb = c.meta_base[rh];
    for (int i = wid; i < touched; i += kSelWaves) {
      const int p = p_first + i;
      const int phys = pg[i];
      const int64_t meta = mb + p;
      if (phys < 0 || meta < 0 || meta >= c.num_meta) continue;
      const int lo_pos = max(n, p * P), hi_pos = min(n + q, (p + 1) * P);
      float lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = __builtin_inff();
        hi[e] = -__builtin_inff();
      }
      uint4 rows[TL];
#pragma unroll
      for (int k = 0; k < TL; ++k) {   // row rg + RPL k of the page, clamped into the chunk's rows
        const int pos = min(max(p * P + rg + RPL * k, lo_pos), hi_pos - 1);
        rows[k] = ld16(ksrc + (int64_t)kept[pos - n] * D + 8 * col);
      }
#pragma unroll
      for (int k = 0; k < TL; ++k) {
        const int pos = p * P + rg + RPL * k;
        if (pos < lo_pos || pos >= hi_pos) continue;
        const uint32_t w[4] = {rows[k].x, rows[k].y, rows[k].z, rows[k].w};
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
      if (rg == 0) {
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
  }
  if (tid == 0) c.seq_len[rh] = n + q;
}

template <int D, typename DT>
hipError_t launch_d(const CacheView& c, const void* k_chunk, const void* v_chunk,
                    const float* scores, const int32_t* quota, int C, hipStream_t s) {
  constexpr int P = 16;
  const size_t lds = (size_t)C * (sizeof(uint32_t) + sizeof(uint16_t)) +
                     (size_t)(C / P + 2) * sizeof(int);
  hipLaunchKernelGGL((prefill_kernel<D, DT>), dim3((unsigned)(c.b * c.Hkv)), dim3(kSelThreads), lds,
                     s, c, static_cast<const uint16_t*>(k_chunk),
                     static_cast<const uint16_t*>(v_chunk), scores, quota, C);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const CacheView& c, const void* k_chunk, const void* v_chunk,
                          const float* scores, const int32_t* quota, int C, hipStream_t s) {
  if (c.dtype == KVS_F16)
    return c.d == 128 ? launch_d<128, F16>(c, k_chunk, v_chunk, scores, quota, C, s)
                      : launch_d<256, F16>(c, k_chunk, v_chunk, scores, quota, C, s);
  return c.d == 128 ? launch_d<128, BF16>(c, k_chunk, v_chunk, scores, quota, C, s)
                    : launch_d<256, BF16>(c, k_chunk, v_chunk, scores, quota, C, s);
}

}  // namespace kvs
