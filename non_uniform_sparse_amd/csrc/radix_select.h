// Block-wide selection of the k largest of n fp32 values, shared by the
// top-K page selection and the per-chunk token selection of a chunked
// prefill.  One block of 256 threads: the values become order-preserving
// 32-bit keys held in LDS; a most-significant-digit radix select (4 passes of
// 8 bits) finds the k-th largest key tau.  A pass whose candidate keys (those
// matching the digits chosen so far) all share one digit takes it directly;
// otherwise it builds a 256-bin LDS histogram of the candidates, one wave
// owns the bins (4 per lane), a suffix scan over its lanes gives the count
// above each lane's bins and the one lane whose bins straddle the k-th key
// publishes the digit.  Items with key > tau are kept, and among items with
// key == tau the lowest indices fill the remaining places.  To place them,
// each thread owns one contiguous run of items and counts its keys above and
// equal to tau; one block-wide exclusive scan of the two counts (packed in
// one int) gives each thread its first output position and the ties taken
// before it, and the thread emits its kept items in index order.  Integer
// work only, so the result is deterministic.
#pragma once

#include "kvs_device.h"

namespace kvs {
namespace {

// Larger float -> larger key; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;

// Block-wide exclusive prefix sum of one int per thread, in thread order.
__device__ __forceinline__ int block_exclusive_scan(int v, int* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) red[wid] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) before += w < wid ? red[w] : 0;
  __syncthreads();
  return before + incl - v;
}

// Block-wide min and max of one int per thread (every thread gets both).
__device__ __forceinline__ void block_minmax(int lo, int hi, int* red, int* out_lo, int* out_hi) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  lo = -(int)group_max<64>(-(float)lo);
  hi = (int)group_max<64>((float)hi);
  if (lane == 0) {
    red[wid] = lo;
    red[kSelWaves + wid] = hi;
  }
  __syncthreads();
  int a = red[0], b = red[kSelWaves];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) {
    a = min(a, red[w]);
    b = max(b, red[kSelWaves + w]);
  }
  __syncthreads();
  *out_lo = a;
  *out_hi = b;
}

// Block-shared scratch of a selection.
struct SelectShared {
  int hist[256];
  int red[2 * kSelWaves];
  int digit, need;
};

struct Threshold {
  uint32_t tau;   // the k-th largest key
  int ties;       // items with key == tau that are kept
};

// keys[i] = order_key(values[i]) for i < n.  All of a thread's loads are
// issued before the first store, so a long row costs one memory round trip
// per 4096 values, not one per 256.  Ends with a barrier.
__device__ void load_keys(const float* __restrict__ values, int n, uint32_t* keys) {
  const int tid = threadIdx.x;
  constexpr int CH = 16;
  for (int base = 0; base < n; base += kSelThreads * CH) {
    float v[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) v[j] = values[min(base + j * kSelThreads + tid, n - 1)];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int p = base + j * kSelThreads + tid;
      if (p < n) keys[p] = order_key(v[j]);
    }
  }
  __syncthreads();
}

// The count-th largest of the n keys (1 <= count <= n; for count = 0 the
// result is not used).  Every thread of the block calls it (it holds
// barriers).
__device__ Threshold kth_largest(const uint32_t* keys, int n, int count, SelectShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int npg = n, keep = count;
  int* hist = sh.hist;
  int* red = sh.red;
  uint32_t prefix = 0, mask = 0;
  int need = keep;   // keys equal to the final prefix still to take
  for (int shift = 24; shift >= 0 && keep > 0; shift -= 8) {
    // Scores of one head often share their top bits: if every candidate key
    // has the same digit, it is the digit, with no histogram (and no atomic
    // contention on one bin).
    int dmin = 256, dmax = -1;
#pragma unroll 4
    for (int p = tid; p < npg; p += kSelThreads) {
      const uint32_t k = keys[p];
      if ((k & mask) == prefix) {
        const int dg = (int)((k >> shift) & 255u);
        dmin = min(dmin, dg);
        dmax = max(dmax, dg);
      }
    }
    block_minmax(dmin, dmax, red, &dmin, &dmax);
    if (dmin == dmax) {
      prefix |= (uint32_t)dmin << shift;
      mask |= 255u << shift;
      continue;
    }
    hist[tid] = 0;   // kSelThreads == 256 bins
    __syncthreads();
#pragma unroll 4
    for (int p = tid; p < npg; p += kSelThreads) {
      const uint32_t k = keys[p];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    if (wid == 0) {
      int hb[4], mine = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hb[i] = hist[4 * lane + i];
        mine += hb[i];
      }
      // inclusive suffix sum over lanes (lane 63 holds the largest digits)
      int incl = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += t;
      }
      int acc = incl - mine;   // keys in bins above this lane's
      int found = -1, left = 0;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (found < 0 && acc < need && need <= acc + hb[i]) {
          found = 4 * lane + i;
          left = need - acc;
        }
        acc += hb[i];
      }
      if (found >= 0) {   // exactly one lane
        sh.digit = found;
        sh.need = left;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh.digit << shift;
    need = sh.need;
    mask |= 255u << shift;
    __syncthreads();
  }
  return Threshold{prefix, need};
}

// Calls emit(pos, i) for each of the count kept items, pos = 0..count-1 in
// index order.  Every thread of the block calls it (it holds barriers).
template <typename Emit>
__device__ void place_kept(const uint32_t* keys, int n, int count, Threshold th, SelectShared& sh,
                           Emit emit) {
  const int tid = threadIdx.x;
  const int npg = n, keep = count;
  const uint32_t tau = th.tau;
  const int ties = th.ties;
  int* red = sh.red;
  // Thread tid owns items [p_lo, p_hi): count keys above and equal to tau
  // (each count < 2^14 since n <= 8192), scan, then place.
  if (keep > 0) {
    const int per = (npg + kSelThreads - 1) / kSelThreads;
    const int p_lo = min(npg, tid * per), p_hi = min(npg, p_lo + per);
    int n_gt = 0, n_eq = 0;
    for (int p = p_lo; p < p_hi; ++p) {
      const uint32_t k = keys[p];
      n_gt += k > tau;
      n_eq += k == tau;
    }
    const int before = block_exclusive_scan((n_gt << 16) | n_eq, red);
    const int gt_before = before >> 16, eq_before = before & 0xffff;
    int pos = gt_before + min(eq_before, ties);
    int eq_seen = eq_before;
    for (int p = p_lo; p < p_hi; ++p) {
      const uint32_t k = keys[p];
      const bool eq = k == tau;
      const bool take = k > tau || (eq && eq_seen < ties);
      eq_seen += eq;
      if (take) {
        if (pos < keep) emit(pos, p);
        ++pos;
      }
    }
  }
}

}  // namespace
}  // namespace kvs
