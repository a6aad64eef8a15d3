// Ragged split-K flash-decode over head-group page tables, and the
// log-sum-exp combine of the splits (FlexiCache summary, Core method: sparse
// flash-decoding over each head's selected pages; Tangram review, 3.2 Ragged
// Paging and 3.3 AOT Load Balancing: per-group tables and a static split map
// S with S_i workgroups for group i).
//
// Work decomposition.  For request r and group i the units are (slot, page)
// pairs, head-major: all attended pages of slot 0, then slot 1, ...  With U
// units and S_i splits, split s owns units [floor(s U/S_i), floor((s+1) U/S_i)).
// One 64-lane workgroup (one wave) per (r, i, s) walks its units in order,
// keeping an online softmax per query head of the KV head it is in, and
// emits a partial (o, lse) for every head it touched.  The combine kernel
// finds, for each query head, the contiguous splits that touched its KV head
// and merges them.
//
// Lane layout for one page of one head (P = 16 rows of d 16-bit elements):
// lane l takes channels 8*(l % COLS) .. +8 of rows rg + RPL*k, rg = l / COLS,
// k < TL, with COLS = d/8, RPL = 64/COLS, TL = 16/RPL.  Every load
// instruction reads RPL whole rows (1 KB), so the 4 KB (d=128) or 8 KB
// (d=256) K and V tiles stream in fully coalesced 16-byte accesses.  Logits
// are pair-dots of q with K summed over the row's COLS lanes; p*V is
// accumulated per lane and reduced over the row groups once per head.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int P = 16;

struct GroupUnits {
  int head[kMaxHp];    // KV head in each slot (-1 = empty slot)
  int count[kMaxHp];   // attended pages of each slot
  int start[kMaxHp];   // first unit of each slot
  int total;
};

// Heads and unit counts of group gi of request r, identical in both kernels.
__device__ void group_units(const DecodeArgs& a, int r, int gi, GroupUnits* gu) {
  const CacheView& c = a.c;
  const int lane = threadIdx.x;
  if (lane < kMaxHp) gu->head[lane] = -1;
  __syncthreads();
  for (int h = lane; h < c.Hkv; h += 64) {
    const int hs = c.head_slot[h];
    if (hs >= 0 && hs < c.Hkv && hs / c.Hp == gi) gu->head[hs % c.Hp] = h;
  }
  __syncthreads();
  if (lane < c.Hp) {
    const int h = gu->head[lane];
    int cnt = 0;
    if (h >= 0) {
      const int n = clampi(c.seq_len[r * c.Hkv + h], 0, P * c.maxpg);
      cnt = (n + P - 1) / P;
      if (a.sel) cnt = min(cnt, clampi(a.sel_count[r * c.Hkv + h], 0, a.K));
    }
    gu->count[lane] = cnt;
  }
  __syncthreads();
  if (lane == 0) {
    int acc = 0;
    for (int j = 0; j < c.Hp; ++j) {
      gu->start[j] = acc;
      acc += gu->count[j];
    }
    gu->total = acc;
  }
  __syncthreads();
}

template <int D, int GQ, typename DT>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  constexpr int COLS = D / 8;
  constexpr int RPL = 64 / COLS;
  constexpr int TL = P / RPL;
  __shared__ GroupUnits gu;
  const CacheView& c = a.c;
  const int lane = threadIdx.x;
  const int r = blockIdx.x / a.splits_total;
  const int rem = blockIdx.x % a.splits_total;
  int gi = 0;
  while (rem >= a.S_prefix[gi + 1]) ++gi;
  const int Si = a.S_prefix[gi + 1] - a.S_prefix[gi];
  const int s = rem - a.S_prefix[gi];

  group_units(a, r, gi, &gu);
  const int64_t U = gu.total;
  const int u0 = (int)((int64_t)s * U / Si), u1 = (int)((int64_t)(s + 1) * U / Si);
  if (u0 >= u1) return;

  const int rg = lane / COLS, col = lane % COLS;
  const int32_t* pt = c.page_table + ((int64_t)r * c.G + gi) * c.maxpg;
  const uint16_t* kvb = reinterpret_cast<const uint16_t*>(c.kv);
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q);

  for (int j = 0; j < c.Hp; ++j) {
    const int a0 = max(u0, gu.start[j]), a1 = min(u1, gu.start[j] + gu.count[j]);
    if (a0 >= a1) continue;
    const int h = gu.head[j];
    const int n = clampi(c.seq_len[r * c.Hkv + h], 0, P * c.maxpg);
    const int32_t* srow = a.sel ? a.sel + ((int64_t)r * c.Hkv + h) * a.K : nullptr;

    uint32_t qw[GQ][4];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const uint4 v = ld16(qb + ((int64_t)r * c.Hq + h * GQ + g) * D + 8 * col);
      qw[g][0] = v.x;
      qw[g][1] = v.y;
      qw[g][2] = v.z;
      qw[g][3] = v.w;
    }
    float m[GQ], l[GQ], o[GQ][8];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      m[g] = -__builtin_inff();
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
    }

    for (int u = a0; u < a1; ++u) {
      const int lp = srow ? srow[u - gu.start[j]] : u - gu.start[j];
      if (lp < 0 || lp >= c.maxpg) continue;
      const int phys = pt[lp];
      if (phys < 0 || phys >= c.num_pages) continue;
      const int valid = min(P, n - lp * P);
      if (valid <= 0) continue;
      const uint16_t* kt = kvb + ((int64_t)phys * c.Hp + j) * 2 * P * D;
      const uint16_t* vt = kt + P * D;
      uint4 kr[TL], vr[TL];
#pragma unroll
      for (int k = 0; k < TL; ++k) kr[k] = ld16(kt + (rg + RPL * k) * D + 8 * col);
#pragma unroll
      for (int k = 0; k < TL; ++k) vr[k] = ld16(vt + (rg + RPL * k) * D + 8 * col);

      float z[TL][GQ];
#pragma unroll
      for (int k = 0; k < TL; ++k) {
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
          float acc = dot2(qw[g][0], kr[k].x, 0.f, DT());
          acc = dot2(qw[g][1], kr[k].y, acc, DT());
          acc = dot2(qw[g][2], kr[k].z, acc, DT());
          acc = dot2(qw[g][3], kr[k].w, acc, DT());
          z[k][g] = group_sum<COLS>(acc);
        }
      }
#pragma unroll
      for (int k = 0; k < TL; ++k) {
        const bool ok = rg + RPL * k < valid;
#pragma unroll
        for (int g = 0; g < GQ; ++g) z[k][g] = ok ? z[k][g] * a.scale_log2 : -__builtin_inff();
        if (!ok) vr[k] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        float tmax = z[0][g];
#pragma unroll
        for (int k = 1; k < TL; ++k) tmax = fmaxf(tmax, z[k][g]);
        tmax = across_max<COLS>(tmax);
        const float mnew = fmaxf(m[g], tmax);
        const float corr = exp2f(m[g] - mnew);
        m[g] = mnew;
        l[g] *= corr;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] *= corr;
#pragma unroll
        for (int k = 0; k < TL; ++k) {
          const float pk = exp2f(z[k][g] - mnew);
          l[g] += pk;
          const uint32_t w[4] = {vr[k].x, vr[k].y, vr[k].z, vr[k].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[g][2 * e] += pk * lo_f(w[e], DT());
            o[g][2 * e + 1] += pk * hi_f(w[e], DT());
          }
        }
      }
    }

    // Merge the row groups and write this split's partial for head h.
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      l[g] = across_sum<COLS>(l[g]);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = across_sum<COLS>(o[g][e]);
    }
    if (rg == 0) {
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        const int64_t row = ((int64_t)r * c.Hq + h * GQ + g) * a.Smax + s;
        const bool empty = !(l[g] > 0.f);
        const float inv = empty ? 0.f : 1.f / l[g];
        float4* dst = reinterpret_cast<float4*>(a.o_part + row * D + 8 * col);
        dst[0] = make_float4(o[g][0] * inv, o[g][1] * inv, o[g][2] * inv, o[g][3] * inv);
        dst[1] = make_float4(o[g][4] * inv, o[g][5] * inv, o[g][6] * inv, o[g][7] * inv);
        if (col == 0) a.lse_part[row] = empty ? -__builtin_inff() : m[g] + log2f(l[g]);
      }
    }
  }
}

// Split that owns unit u when U units are cut into S ranges starting at
// floor(s U / S): the largest s with floor(s U / S) <= u, i.e.
// s = floor(((u + 1) S - 1) / U).
__device__ __forceinline__ int split_of(int64_t u, int64_t U, int64_t S) {
  return (int)(((u + 1) * S - 1) / U);
}

template <int D>
__global__ __launch_bounds__(64) void combine_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;   // channels per lane
  __shared__ GroupUnits gu;
  const CacheView& c = a.c;
  const int lane = threadIdx.x;
  const int r = blockIdx.x / c.Hq;
  const int g = blockIdx.x % c.Hq;
  const int h = g / c.Gq;
  const int hs = c.head_slot[h];
  float* dst = a.out + ((int64_t)r * c.Hq + g) * D;
  if (hs < 0 || hs >= c.Hkv) {
    for (int e = lane; e < D; e += 64) dst[e] = 0.f;
    return;
  }
  const int gi = hs / c.Hp, j = hs % c.Hp;
  group_units(a, r, gi, &gu);
  const int64_t U = gu.total;
  const int Si = a.S_prefix[gi + 1] - a.S_prefix[gi];
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  if (gu.count[j] > 0) {
    const int s_lo = split_of(gu.start[j], U, Si);
    const int s_hi = split_of(gu.start[j] + gu.count[j] - 1, U, Si);
    const int64_t row = ((int64_t)r * c.Hq + g) * a.Smax;
    // A split whose unit range is empty wrote nothing (possible when U < S_i).
    auto nonempty = [&](int64_t s) { return (s * U) / Si < ((s + 1) * U) / Si; };
    float M = -__builtin_inff();
    for (int s = s_lo; s <= s_hi; ++s)
      if (nonempty(s)) M = fmaxf(M, a.lse_part[row + s]);
    if (M > -__builtin_inff()) {
      float den = 0.f;
      for (int s = s_lo; s <= s_hi; ++s) {
        if (!nonempty(s)) continue;
        const float w = exp2f(a.lse_part[row + s] - M);
        den += w;
        const float* src = a.o_part + (row + s) * D;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += w * src[lane * PER + e];
      }
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] /= den;
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[lane * PER + e] = acc[e];
}

template <int D, int GQ, typename DT>
hipError_t launch_decode_v(const DecodeArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.c.b * a.splits_total;
  hipLaunchKernelGGL((decode_kernel<D, GQ, DT>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int D, typename DT>
hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
  switch (a.c.Gq) {
    case 1: return launch_decode_v<D, 1, DT>(a, s);
    case 2: return launch_decode_v<D, 2, DT>(a, s);
    case 4: return launch_decode_v<D, 4, DT>(a, s);
    default: return launch_decode_v<D, 8, DT>(a, s);
  }
}

template <int D, int GQ, typename DT>
const void* decode_symbol() {
  return reinterpret_cast<const void*>(&decode_kernel<D, GQ, DT>);
}

template <int D, typename DT>
const void* decode_symbol_g(int gqa) {
  switch (gqa) {
    case 1: return decode_symbol<D, 1, DT>();
    case 2: return decode_symbol<D, 2, DT>();
    case 4: return decode_symbol<D, 4, DT>();
    default: return decode_symbol<D, 8, DT>();
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.c.dtype == KVS_F16)
    return a.c.d == 128 ? launch_decode_g<128, F16>(a, s) : launch_decode_g<256, F16>(a, s);
  return a.c.d == 128 ? launch_decode_g<128, BF16>(a, s) : launch_decode_g<256, BF16>(a, s);
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.c.b * a.c.Hq;
  if (a.c.d == 128)
    hipLaunchKernelGGL((combine_kernel<128>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((combine_kernel<256>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t decode_blocks_per_cu(int d, int gqa, int dtype, int* blocks) {
  const void* fn;
  if (dtype == KVS_F16)
    fn = d == 128 ? decode_symbol_g<128, F16>(gqa) : decode_symbol_g<256, F16>(gqa);
  else
    fn = d == 128 ? decode_symbol_g<128, BF16>(gqa) : decode_symbol_g<256, BF16>(gqa);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, fn, 64, 0);
}

}  // namespace kvs
