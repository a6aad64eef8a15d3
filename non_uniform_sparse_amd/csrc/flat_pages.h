// Even division of all heads' pages over a resident-sized grid, shared by
// the kernels that stream every page of every head (min-max build, page
// scores).  Heads hold from a few to thousands of pages, so a grid of one
// wave per fixed chunk of one head leaves most waves idle or short-lived;
// instead each block forms the prefix sum of the heads' page counts in LDS
// and wave w of W takes flat pages [T*w/W, T*(w+1)/W) of the T in all
// heads, walking them as one segment per head it touches.
#pragma once

#include <atomic>

#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kFlatThreads = 256;

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// pre[i] = sum of count(j) over heads j < i, for i in [0, BH]; pre[BH] is
// the total.  count(i) gives head i's page count.  The counts are first
// loaded into pre[] with coalesced loads, up to 8 in flight per thread, then
// summed per contiguous chunk, scanned, and overwritten in place.  Every
// thread of the block calls this (it holds barriers).
template <typename Count>
__device__ void page_prefix(int BH, Count count, int* pre, int* part) {
  const int tid = threadIdx.x;
  constexpr int CH = 8;
  for (int base = 0; base < BH; base += kFlatThreads * CH) {
    int v[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) v[j] = count(min(base + j * kFlatThreads + tid, BH - 1));
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int i = base + j * kFlatThreads + tid;
      if (i < BH) pre[i] = v[j];
    }
  }
  __syncthreads();
  const int per = (BH + kFlatThreads - 1) / kFlatThreads;
  const int lo = min(BH, tid * per), hi = min(BH, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += pre[i];
  part[tid] = s;
  __syncthreads();
  if (tid < 64) {   // exclusive scan of the 256 partial sums, 4 per lane
    int v[4], t = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = part[4 * tid + k];
      t += v[k];
    }
    int incl = t;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int n = __shfl_up(incl, off, 64);
      if (tid >= off) incl += n;
    }
    int run = incl - t;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      part[4 * tid + k] = run;
      run += v[k];
    }
  }
  __syncthreads();
  int run = part[tid];
  for (int i = lo; i < hi; ++i) {
    const int n = pre[i];
    pre[i] = run;
    run += n;
  }
  if (tid == kFlatThreads - 1) pre[BH] = run;
  __syncthreads();
}

// This wave's share [t0, t1) of the T flat pages, and the head holding t0
// (the largest hh with pre[hh] <= t0, which is non-empty when t0 < T).
struct FlatShare {
  int t0, t1, hh;
};

__device__ __forceinline__ FlatShare flat_share(const int* pre, int BH) {
  const int64_t W = (int64_t)gridDim.x * (kFlatThreads / 64);
  const int64_t w = (int64_t)blockIdx.x * (kFlatThreads / 64) + uni(threadIdx.x >> 6);
  const int64_t T = uni(pre[BH]);
  FlatShare s;
  s.t0 = uni((int)(T * w / W));
  s.t1 = uni((int)(T * (w + 1) / W));
  int lo = 0, hi = BH;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (uni(pre[mid]) <= s.t0) lo = mid; else hi = mid - 1;
  }
  s.hh = lo;
  return s;
}

// Resident blocks of kFlatThreads threads for `kernel` on the current
// device (compute units x blocks per unit, at most max_per_cu per unit),
// the occupancy found once per device.
template <const void* (*Sym)()>
hipError_t resident_grid(int* grid, int max_per_cu = 1 << 20) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus_of[kMaxDevices], per_cu_of[kMaxDevices];
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int cus = cus_of[dev].load(std::memory_order_relaxed);
  int per_cu = per_cu_of[dev].load(std::memory_order_relaxed);
  if (cus == 0 || per_cu == 0) {
    if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev))
      return e;
    if (hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Sym(), kFlatThreads, 0))
      return e;
    cus = max(1, cus);
    per_cu = max(1, per_cu);
    per_cu_of[dev].store(per_cu, std::memory_order_relaxed);
    cus_of[dev].store(cus, std::memory_order_relaxed);
  }
  *grid = cus * max(1, min(per_cu, max_per_cu));
  return hipSuccess;
}

}  // namespace
}  // namespace kvs
