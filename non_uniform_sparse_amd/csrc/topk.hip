// Per-KV-head top-K page selection (FlexiCache summary, Core method: each
// head attends only its K best pages).  One 256-thread workgroup per
// (request, head).  Scores become order-preserving 32-bit keys held in LDS;
// a most-significant-digit radix select (4 passes of 8 bits, LDS histogram)
// finds the K-th largest key tau; pages with key > tau are kept, and among
// pages with key == tau the lowest page indices fill the remaining places.
// Two block-wide exclusive scans in page order (equal keys, then kept pages)
// rank the ties and place the kept pages in ascending page order.  Integer
// work only, so the result is deterministic.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;

// Larger float -> larger key; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one int per thread over the workgroup; returns the
// thread's prefix and writes the total to *total.
__device__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int tid = threadIdx.x;
  lds[tid] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = tid >= off ? lds[tid - off] : 0;
    __syncthreads();
    lds[tid] += add;
    __syncthreads();
  }
  const int incl = lds[tid];
  *total = lds[kThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ seq_len, int P,
                                                        int Hkv, int max_pages, int K,
                                                        int32_t* __restrict__ sel,
                                                        int32_t* __restrict__ sel_count) {
  __shared__ uint32_t keys[kMaxTopkPages];
  __shared__ int hist[256];
  __shared__ int scan[kThreads];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;

  const int rh = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = clampi(seq_len[rh], 0, P * max_pages);
  const int npg = (n + P - 1) / P;
  const int keep = min(K, npg);
  const float* row = scores + (int64_t)rh * max_pages;
  int32_t* out = sel + (int64_t)rh * K;

  for (int p = tid; p < npg; p += kThreads) keys[p] = order_key(row[p]);
  if (tid == 0) {
    s_prefix = 0;
    s_need = keep;
  }
  __syncthreads();

  // Radix select of the keep-th largest key.
  uint32_t mask = 0;
  for (int shift = 24; shift >= 0 && keep > 0; shift -= 8) {
    hist[tid] = 0;  // kThreads == 256 bins
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int p = tid; p < npg; p += kThreads) {
      const uint32_t k = keys[p];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int need = s_need, digit = 255;
      for (; digit > 0; --digit) {
        if (hist[digit] >= need) break;
        need -= hist[digit];
      }
      s_prefix = prefix | ((uint32_t)digit << shift);
      s_need = need;
    }
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t tau = s_prefix;
  const int ties = s_need;   // pages equal to tau still to take

  // Contiguous page range of this thread, in page order.
  const int per = (npg + kThreads - 1) / kThreads;
  const int p0 = min(npg, tid * per), p1 = min(npg, p0 + per);
  int eq = 0;
  for (int p = p0; p < p1; ++p) eq += keys[p] == tau;
  int total;
  int eq_before = block_exclusive_scan(eq, scan, &total);
  int kept = 0;
  for (int p = p0; p < p1; ++p) {
    const uint32_t k = keys[p];
    if (k > tau || (k == tau && eq_before++ < ties)) ++kept;
  }
  int pos = block_exclusive_scan(kept, scan, &total);
  eq_before -= eq;   // rewind to this range's first tie rank
  if (keep > 0) {
    for (int p = p0; p < p1; ++p) {
      const uint32_t k = keys[p];
      if (k > tau || (k == tau && eq_before++ < ties)) out[pos++] = p;
    }
  }
  for (int k = keep + tid; k < K; k += kThreads) out[k] = -1;
  if (tid == 0) sel_count[rh] = keep;
}

}  // namespace

hipError_t launch_topk(const float* scores, const int32_t* seq_len, int P, int b, int Hkv,
                       int max_pages, int K, int32_t* sel, int32_t* sel_count, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)(b * Hkv)), dim3(kThreads), 0, s, scores, seq_len,
                     P, Hkv, max_pages, K, sel, sel_count);
  return hipGetLastError();
}

}  // namespace kvs
