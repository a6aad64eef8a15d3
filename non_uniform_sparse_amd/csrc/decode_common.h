// Pieces of the split-K decode kernel: the unit bookkeeping of one
// (request, group) and the lane geometry and math of a page.
#pragma once

#include <utility>

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

// Heads and unit counts of group gi of request r.  Lane h reads head h's
// slot, length and selection count at once (no load waits on another), and
// the heads of group gi fill their slots' entries.
__device__ void group_units(const DecodeArgs& a, int r, int gi, GroupUnits* gu) {
  const CacheView& c = a.c;
  const int lane = threadIdx.x;
  if (lane < kMaxHp) {
    gu->head[lane] = -1;
    gu->count[lane] = 0;
  }
  __syncthreads();
  for (int h = lane; h < c.Hkv; h += 64) {
    const int hs = c.head_slot[h];
    const int n = clampi(c.seq_len[r * c.Hkv + h], 0, P * c.maxpg);
    const int sc = a.sel ? a.sel_count[r * c.Hkv + h] : 0;
    if (hs >= 0 && hs < c.Hkv && hs / c.Hp == gi) {
      int cnt = (n + P - 1) / P;
      if (a.sel) cnt = min(cnt, clampi(sc, 0, a.K));
      gu->head[hs % c.Hp] = h;
      gu->count[hs % c.Hp] = cnt;
    }
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

// ---------------------------------------------------------------------------
// Per-page math.  Logits of the page's 16 tokens against the GQ query heads
// form a small dense contraction, S^T[16 tokens][16 cols] = K[16][d] Q^T[d][16]
// (cols >= GQ are zero), done as d/32 v_mfma_f32_16x16x32 steps.  MFMA lane
// layouts (gfx950): A operand lane l holds A[l%16][8(l/16)..+8] of each 32-wide
// k block, B operand B[8(l/16)..+8][l%16], result D[4(l/16)+i][l%16], i < 4.
// MFMA row m is mapped to token tau(m) so that the result lands where the p*V
// step needs it: the V side gives lane l the channels 8*(l % COLS)..+8 of rows
// rg + RPL*k (rg = l / COLS, k < TL), and the result lane of column g in row
// group a = rg*A + hh (A = 4/RPL, hh < A) holds tokens rg + RPL*(4 hh + i).
// Softmax statistics live in the result layout (each lane tracks the query
// head of its column); probabilities and rescale factors reach the V lanes
// through ds_swizzle row broadcasts.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c, F16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c, BF16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ds_swizzle bit-mask mode within 32-lane halves: source = (lane & and) | or.
template <int AND, int OR>
__device__ __forceinline__ float swz(float v) {
  return __uint_as_float(__builtin_amdgcn_ds_swizzle(__float_as_uint(v), (OR << 5) | AND));
}

template <int D>
struct Geometry {
  static constexpr int COLS = D / 8;        // V lanes per row (8 channels each)
  static constexpr int RPL = 64 / COLS;     // V row groups
  static constexpr int TL = P / RPL;        // rows per V lane
  static constexpr int A = 4 / RPL;         // result row groups per V row group
  static constexpr int KB = D / 32;         // MFMA k blocks
};

// Value held by result lane (row group rg*A + HH, column G) broadcast to every
// lane of V row group rg.
template <int D, int HH, int G>
__device__ __forceinline__ float from_result(float v) {
  constexpr int A = Geometry<D>::A;
  if constexpr (A == 1) return swz<0x10, G>(v);      // rows of 16; keep lane bit 4
  else return swz<0x00, 16 * HH + G>(v);             // two result rows per 32-lane half
}

// Measurement build only (libkvs_valu.so): the page's logits as VALU
// pair-dot products summed across each row's lanes instead of MFMA, the
// rest unchanged -- the comparison that justifies MFMA for the query
// group's logits.
#ifdef KVS_VALU_LOGITS
constexpr bool kValuLogits = true;
#else
constexpr bool kValuLogits = false;
#endif

// Attention of one wave over pages of one KV head: the lane roles, the
// head's query operand and running softmax state, and the per-page step
// (FlexiCache summary, Core method: flash-decoding over a head's pages).
// A page is the head's P x D K tile and V tile; the wave loads both in the
// coalesced V-side layout (load_k / load_v: RPL whole rows per
// instruction, non-temporal), stages K through LDS into the MFMA operand
// layout, forms the logits of the page's 16 tokens against the GQ query
// rows with MFMA, keeps the online softmax in the result layout, and
// accumulates p*V on the VALU in the V layout.
template <int D, int GQ, typename DT>
struct PageAttention {
  using Geo = Geometry<D>;
  static constexpr int COLS = Geo::COLS, RPL = Geo::RPL, TL = Geo::TL, A = Geo::A, KB = Geo::KB;
  static constexpr int KROW = D + 8;   // LDS row stride (halves): 16 B pad
  static constexpr int KTILE_HALVES = P * KROW;
  static_assert(GQ <= 16, "query group must fit the 16 MFMA columns");

  int rg, vcol, v_off;           // V side (also how K is fetched)
  int kq, k_lds, w_lds;          // MFMA operand roles
  int rcol, r_tok0;              // result roles: column (query row), first token
  uint4 qop[KB];                 // Q^T operand of the current head
  float m_col, l_col;            // running max / partial sum of column rcol
  float o[GQ][8];                // V-side accumulators
  uint32_t qv[GQ][4];            // VALU logits only: this lane's 8 channels of each query row
  float m_v[GQ], l_v[GQ];        // VALU logits only: running max / partial sum per query row

  __device__ explicit PageAttention(int lane) {
    rg = lane / COLS;
    vcol = lane % COLS;
    v_off = rg * D + 8 * vcol;
    // MFMA roles: operand row m = lane % 16 (a token), k sub-block kq = lane / 16
    const int m = lane % 16;
    kq = lane / 16;
    const int ka = m / 4, ki = m % 4;
    const int k_tok = (ka / A) + RPL * (4 * (ka % A) + ki);   // token fed as MFMA row m
    k_lds = k_tok * KROW + 8 * kq;                            // its operand slice in LDS
    w_lds = rg * KROW + 8 * vcol;                             // where this lane stores K rows
    // result role: column (query head) rcol, row group ra holding 4 tokens
    rcol = lane % 16;
    const int ra = lane / 16;
    r_tok0 = (ra / A) + RPL * 4 * (ra % A);                   // token of element i: r_tok0 + RPL*i
  }

  __device__ __forceinline__ void load_k(const uint16_t* tile, uint4 (&dst)[TL]) const {
#pragma unroll
    for (int k = 0; k < TL; ++k) dst[k] = ld16_once(tile + v_off + RPL * k * D);
  }
  __device__ __forceinline__ void load_v(const uint16_t* tile, uint4 (&dst)[TL]) const {
#pragma unroll
    for (int k = 0; k < TL; ++k) dst[k] = ld16_once(tile + P * D + v_off + RPL * k * D);
  }

  // Starts a head: q_head points at its first query row ([GQ][D]).
  __device__ __forceinline__ void begin(const uint16_t* q_head) {
    const bool has = rcol < GQ;
    // unconditional loads (columns >= GQ read row 0 and are zeroed), so no
    // branch hides them from the wait-count bookkeeping of the loop
    const uint16_t* qrow = q_head + (has ? rcol : 0) * D + 8 * kq;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint4 v = ld16(qrow + 32 * kb);
      qop[kb] = has ? v : make_uint4(0, 0, 0, 0);
    }
    m_col = -__builtin_inff();
    l_col = 0.f;
#pragma unroll
    for (int g = 0; g < GQ; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
    if constexpr (kValuLogits) {
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        const uint4 v = ld16(q_head + g * D + 8 * vcol);
        qv[g][0] = v.x;
        qv[g][1] = v.y;
        qv[g][2] = v.z;
        qv[g][3] = v.w;
        m_v[g] = -__builtin_inff();
        l_v[g] = 0.f;
      }
    }
  }

  // One page with `valid` >= 1 tokens, its K and V rows in kc / vr.
  // refill_k() runs once the K rows are staged (the K registers are free),
  // refill_v() once p*V is done (the V registers are free): the caller
  // prefetches a later page there.  ktile: LDS of KTILE_HALVES halves.
  template <typename RefillK, typename RefillV>
  __device__ __forceinline__ void page(uint4 (&kc)[TL], uint4 (&vr)[TL], int valid,
                                       uint16_t* ktile, float scale_log2, RefillK refill_k,
                                       RefillV refill_v) {
    float cg[GQ], pb[TL][GQ];   // rescale factor per query head, probabilities per V row
    if constexpr (kValuLogits) {
      // logits of the lane's rows: pair-dots over its 8 channels, summed
      // across the row's COLS lanes; softmax in the V layout
      float z[TL][GQ];
#pragma unroll
      for (int k = 0; k < TL; ++k) {
        const bool ok = rg + RPL * k < valid;
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
          float acc = dot2(qv[g][0], kc[k].x, 0.f, DT());
          acc = dot2(qv[g][1], kc[k].y, acc, DT());
          acc = dot2(qv[g][2], kc[k].z, acc, DT());
          acc = dot2(qv[g][3], kc[k].w, acc, DT());
          acc = group_sum<COLS>(acc);
          z[k][g] = ok ? acc * scale_log2 : -__builtin_inff();
        }
      }
      refill_k();
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        float tmax = z[0][g];
#pragma unroll
        for (int k = 1; k < TL; ++k) tmax = fmaxf(tmax, z[k][g]);
        tmax = across_max<COLS>(tmax);
        const float mnew = fmaxf(m_v[g], tmax);
        cg[g] = __builtin_amdgcn_exp2f(m_v[g] - mnew);
        m_v[g] = mnew;
        float psum = 0.f;
#pragma unroll
        for (int k = 0; k < TL; ++k) {
          pb[k][g] = __builtin_amdgcn_exp2f(z[k][g] - mnew);
          psum += pb[k][g];
        }
        l_v[g] = l_v[g] * cg[g] + psum;
      }
    } else {
      // K rows -> LDS, then back in MFMA operand layout (the global loads stay
      // whole-row coalesced; the MFMA wants 16 rows x 64 B per operand).
#pragma unroll
      for (int k = 0; k < TL; ++k)
        *reinterpret_cast<uint4*>(ktile + w_lds + RPL * k * KROW) = kc[k];
      refill_k();   // K registers free: fetch a later page's K
      // A wave's LDS operations execute in order; the compiler barrier
      // keeps the reads after the writes and the LDS-only wait (vmcnt,
      // expcnt left at their maxima) leaves the prefetch loads in flight.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);
      uint4 kr[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        kr[kb] = *reinterpret_cast<const uint4*>(ktile + k_lds + 32 * kb);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = mfma16x16x32(kr[kb], qop[kb], acc, DT());
      // online softmax in the result layout (column rcol = query head)
      float z[4], tmax = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = r_tok0 + RPL * i < valid ? acc[i] * scale_log2 : -__builtin_inff();
        tmax = fmaxf(tmax, z[i]);
      }
      tmax = across_max<16>(tmax);
      const float mnew = fmaxf(m_col, tmax);
      const float corr = __builtin_amdgcn_exp2f(m_col - mnew);
      m_col = mnew;
      float pr[4], psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(z[i] - mnew);
        psum += pr[i];
      }
      l_col = l_col * corr + psum;

      // broadcast rescale factors and probabilities to the V lanes
      [&]<int... G>(std::integer_sequence<int, G...>) {
        ((cg[G] = from_result<D, 0, G>(corr)), ...);
        [&]<int... HI>(std::integer_sequence<int, HI...>) {
          auto one = [&]<int HIV>() {
            constexpr int HH = HIV / 4, I = HIV % 4;
            ((pb[4 * HH + I][G] = from_result<D, HH, G>(pr[I])), ...);
          };
          (one.template operator()<HI>(), ...);
        }(std::make_integer_sequence<int, TL>{});
      }(std::make_integer_sequence<int, GQ>{});
    }

#pragma unroll
    for (int g = 0; g < GQ; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] *= cg[g];
#pragma unroll
    for (int k = 0; k < TL; ++k) {
      // rows past the valid count hold no token (possibly NaN): zero them
      const bool ok = rg + RPL * k < valid;
      const uint32_t w[4] = {ok ? vr[k].x : 0u, ok ? vr[k].y : 0u, ok ? vr[k].z : 0u,
                             ok ? vr[k].w : 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = lo_f(w[e], DT()), v1 = hi_f(w[e], DT());
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
          o[g][2 * e] += pb[k][g] * v0;
          o[g][2 * e + 1] += pb[k][g] * v1;
        }
      }
    }
    refill_v();   // V consumed: fetch a later page's V
  }

  // Ends the head: o[g][*] becomes the sum over the V row groups (lanes of
  // row group 0 hold channels 8*vcol .. +8 of query row g), lg[g] the
  // softmax denominator and mg[g] the running max (base 2), uniform.
  __device__ __forceinline__ void finish(float (&lg)[GQ], float (&mg)[GQ]) {
    if constexpr (kValuLogits) {
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        lg[g] = across_sum<COLS>(l_v[g]);   // total over the V row groups
        mg[g] = m_v[g];
      }
    } else {
      const float lt = across_sum<16>(l_col);   // total over the 4 result row groups
      [&]<int... G>(std::integer_sequence<int, G...>) {
        ((lg[G] = from_result<D, 0, G>(lt), mg[G] = from_result<D, 0, G>(m_col)), ...);
      }(std::make_integer_sequence<int, GQ>{});
    }
#pragma unroll
    for (int g = 0; g < GQ; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = across_sum<COLS>(o[g][e]);
  }
};

}  // namespace
}  // namespace kvs
