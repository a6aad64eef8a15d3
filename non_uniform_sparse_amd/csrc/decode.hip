// Ragged split-K flash-decode over head-group page tables (FlexiCache
// summary, Core method: sparse flash-decoding over each head's selected
// pages; Tangram review, 3.2 Ragged Paging and 3.3 AOT Load Balancing:
// per-group tables and a static split map S with S_i workgroups for group
// i).  The log-sum-exp combine of the splits is combine.hip.
//
// Work decomposition.  For request r and group i the units are (slot, page)
// pairs, head-major: all attended pages of slot 0, then slot 1, ...  With U
// units and S_i splits, split s owns units [floor(s U/S_i), floor((s+1) U/S_i)).
// One 64-lane workgroup (one wave) per (r, i, s) walks its units in order,
// keeping an online softmax per query head of the KV head it is in, and
// emits a partial (o, lse) for every head it touched, noting for each head
// whether it is that head's first or last split.  The combine kernel
// (combine.hip) merges, for each query head, the contiguous range of splits
// that touched its KV head.
//
// Lane layout for one page of one head (P = 16 rows of d 16-bit elements):
// lane l takes channels 8*(l % COLS) .. +8 of rows rg + RPL*k, rg = l / COLS,
// k < TL, with COLS = d/8, RPL = 64/COLS, TL = 16/RPL.  Every load
// instruction reads RPL whole rows (1 KB), so the 4 KB (d=128) or 8 KB
// (d=256) K and V tiles stream in fully coalesced 16-byte accesses, marked
// non-temporal (each tile is read once per step).  Logits
// are pair-dots of q with K summed over the row's COLS lanes; p*V is
// accumulated per lane and reduced over the row groups once per head.
#include <algorithm>
#include <utility>

#include "decode_common.h"

namespace kvs {
namespace {

template <int D, int GQ, typename DT>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  using PA = PageAttention<D, GQ, DT>;
  constexpr int COLS = PA::COLS, TL = PA::TL;
  __shared__ GroupUnits gu;
  __shared__ uint4 ktile_raw[PA::KTILE_HALVES / 8];   // one page's K tile, row-major
  uint16_t* ktile = reinterpret_cast<uint16_t*>(ktile_raw);
  const CacheView& c = a.c;
  const int lane = threadIdx.x;
  const int r = blockIdx.x / a.splits_total;
  const int rem = blockIdx.x % a.splits_total;
  int gi = 0;
  while (rem >= a.S_prefix[gi + 1]) ++gi;
  const int Si = a.S_prefix[gi + 1] - a.S_prefix[gi];
  const int s = rem - a.S_prefix[gi];
#ifdef KVS_WG_STAMPS
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  struct Stamp {
    uint64_t* p;
    uint64_t t0;
    __device__ ~Stamp() {
      if (threadIdx.x == 0) {
        p[0] = t0;
        p[1] = __builtin_amdgcn_s_memrealtime();
      }
    }
  } stamp{a.stamps + 2 * (int64_t)blockIdx.x, t_start};
#endif

  group_units(a, r, gi, &gu);
  const int64_t U = gu.total;
  const int u0 = (int)((int64_t)s * U / Si), u1 = (int)((int64_t)(s + 1) * U / Si);
  if (u0 >= u1) {
    // An empty split (U < S_i) that lies strictly inside a head's range of
    // splits marks itself as holding nothing, so the combine can walk the
    // range [first, last] of that head without knowing U.
    if (lane < c.Hp) {
      const int st = gu.start[lane], en = st + gu.count[lane], h = gu.head[lane];
      if (h >= 0 && st < u0 && u0 < en) {
        for (int g = 0; g < GQ; ++g)
          a.lse_part[((int64_t)r * c.Hq + h * GQ + g) * a.Smax + s] = -__builtin_inff();
      }
    }
    return;
  }
  // For each head this split touches: is it the head's first / last split?
  if (lane < c.Hp) {
    const int st = gu.start[lane], en = st + gu.count[lane], h = gu.head[lane];
    if (h >= 0 && gu.count[lane] > 0 && u0 < en && u1 > st) {
      const int64_t hidx = (int64_t)r * c.Hkv + h;
      if (u0 <= st) a.split_lo[hidx] = s;
      if (u1 >= en) a.split_hi[hidx] = s;
    }
  }

  PA pa(lane);
  const int32_t* pt = c.page_table + ((int64_t)r * c.G + gi) * c.maxpg;
  const uint16_t* kvb = reinterpret_cast<const uint16_t*>(c.kv);
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q);
  int cur_j = -1;

  // Merge the row groups and write this split's partial for the head in slot j.
  auto end_head = [&](int j) {
    const int h = gu.head[j];
    float lg[GQ], mg[GQ];
    pa.finish(lg, mg);
    if (pa.rg == 0) {
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        const int64_t row = ((int64_t)r * c.Hq + h * GQ + g) * a.Smax + s;
        const bool empty = !(lg[g] > 0.f);
        const float inv = empty ? 0.f : 1.f / lg[g];
        float4* dst = reinterpret_cast<float4*>(a.o_part + row * D + 8 * pa.vcol);
        dst[0] = make_float4(pa.o[g][0] * inv, pa.o[g][1] * inv, pa.o[g][2] * inv,
                             pa.o[g][3] * inv);
        dst[1] = make_float4(pa.o[g][4] * inv, pa.o[g][5] * inv, pa.o[g][6] * inv,
                             pa.o[g][7] * inv);
        if (pa.vcol == 0) a.lse_part[row] = empty ? -__builtin_inff() : mg[g] + log2f(lg[g]);
      }
    }
  };
  static_assert(COLS * 8 == D, "V lanes cover a row");

  // Pages in flight per wave: two for d = 128 (8 KB pages), one for d = 256
  // (16 KB pages), at the same occupancy.
  constexpr int DEPTH = D == 128 ? 2 : 1;
  uint4 kc[DEPTH][TL], vr[DEPTH][TL];   // K and V rows of upcoming units, coalesced layout
  for (int base = u0; base < u1; base += 64) {
    const int nb = min(64, u1 - base);
    // Lane t resolves unit base + t: its slot, physical page and valid rows.
    int my_j = 0, my_phys = -1, my_valid = 0;
    if (lane < nb) {
      const int u = base + lane;
      int j = 0;
      for (int jj = 1; jj < c.Hp; ++jj)
        if (gu.count[jj] > 0 && u >= gu.start[jj]) j = jj;
      const int h = gu.head[j];
      const int k = u - gu.start[j];
      const int n = clampi(c.seq_len[r * c.Hkv + h], 0, P * c.maxpg);
      const int lp = a.sel ? a.sel[((int64_t)r * c.Hkv + h) * a.K + k] : k;
      if (lp >= 0 && lp < c.maxpg) {
        const int ph = pt[lp];
        if (ph >= 0 && ph < c.num_pages) {
          my_phys = ph;
          my_valid = min(P, n - lp * P);
        }
      }
      my_j = j;
    }
    // Tile of unit t; a missing page reads page 0 instead (always valid
    // memory; such units are skipped), so no load depends on a lane's data.
    auto tile = [&](int t) {
      const int phys = __builtin_amdgcn_readlane(my_phys, t);
      const int j = __builtin_amdgcn_readlane(my_j, t);
      return kvb + (phys >= 0 ? ((int64_t)phys * c.Hp + j) * 2 * P * D : 0);
    };
#pragma unroll
    for (int b = 0; b < DEPTH; ++b) {
      const uint16_t* kt = tile(b < nb ? b : nb - 1);
      pa.load_k(kt, kc[b]);
      pa.load_v(kt, vr[b]);
    }
    // One unit, its tiles in buffer B; refills buffer B with unit t + DEPTH.
    auto unit = [&]<int B>(int t) {
      const int j = __builtin_amdgcn_readlane(my_j, t);
      const int phys = __builtin_amdgcn_readlane(my_phys, t);
      const int valid = __builtin_amdgcn_readlane(my_valid, t);
      if (j != cur_j) {
        if (cur_j >= 0) end_head(cur_j);
        pa.begin(qb + ((int64_t)r * c.Hq + gu.head[j] * GQ) * D);
        cur_j = j;
      }
      // tile to prefetch; past the batch end there is none (the condition is
      // uniform over the wave, and the tiles are read with non-temporal
      // loads, so re-reading the last one would go back to HBM)
      const bool more = t + DEPTH < nb;
      const uint16_t* nt = tile(more ? t + DEPTH : nb - 1);
      if (phys < 0 || valid <= 0) {
        if (more) {
          pa.load_k(nt, kc[B]);
          pa.load_v(nt, vr[B]);
        }
        return;
      }
      pa.page(kc[B], vr[B], valid, ktile, a.scale_log2,
              [&] { if (more) pa.load_k(nt, kc[B]); },
              [&] { if (more) pa.load_v(nt, vr[B]); });
    };
    for (int t0 = 0; t0 < nb; t0 += DEPTH) {
      [&]<int... B>(std::integer_sequence<int, B...>) {
        ((t0 + B < nb ? unit.template operator()<B>(t0 + B) : void()), ...);
      }(std::make_integer_sequence<int, DEPTH>{});
    }
  }
  if (cur_j >= 0) end_head(cur_j);
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

hipError_t decode_blocks_per_cu(int d, int gqa, int dtype, int* blocks) {
  const void* fn;
  if (dtype == KVS_F16)
    fn = d == 128 ? decode_symbol_g<128, F16>(gqa) : decode_symbol_g<256, F16>(gqa);
  else
    fn = d == 128 ? decode_symbol_g<128, BF16>(gqa) : decode_symbol_g<256, BF16>(gqa);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, fn, 64, 0);
}

}  // namespace kvs
