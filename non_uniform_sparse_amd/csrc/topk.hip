// Per-KV-head top-K page selection (FlexiCache summary, Core method: each
// head attends only its K best pages).  One 256-thread workgroup per
// (request, head) runs the block selection of radix_select.h over the
// head's page scores and writes the kept pages in ascending page order;
// entries past the kept count are -1.  A head outside the given set keeps
// the selection it holds.  Integer work only, so the result is
// deterministic.
#include "radix_select.h"
#include "kvs_launch.h"

namespace kvs {
namespace {

__global__ __launch_bounds__(kSelThreads) void topk_kernel(const float* __restrict__ scores,
                                                           const int32_t* __restrict__ seq_len,
                                                           int P, int max_pages, int K, int Hkv,
                                                           HeadMask heads,
                                                           int32_t* __restrict__ sel,
                                                           int32_t* __restrict__ sel_count) {
  extern __shared__ uint32_t keys[];   // [max_pages]
  __shared__ SelectShared sh;
  const int rh = blockIdx.x;
  if (!heads.has(rh % Hkv)) return;   // a head outside the set keeps its selection
  const int tid = threadIdx.x;
  const int n = clampi(seq_len[rh], 0, P * max_pages);
  const int npg = (n + P - 1) / P;
  const int keep = min(K, npg);
  int32_t* out = sel + (int64_t)rh * K;

  load_keys(scores + (int64_t)rh * max_pages, npg, keys);
  const Threshold th = kth_largest(keys, npg, keep, sh);
  place_kept(keys, npg, keep, th, sh, [&](int pos, int p) { out[pos] = p; });
  for (int k = keep + tid; k < K; k += kSelThreads) out[k] = -1;
  if (tid == 0) sel_count[rh] = keep;
}

}  // namespace

hipError_t launch_topk(const float* scores, const int32_t* seq_len, int P, int b, int Hkv,
                       int max_pages, int K, const HeadMask& heads, int32_t* sel,
                       int32_t* sel_count, hipStream_t s) {
  const size_t lds = (size_t)max_pages * sizeof(uint32_t);
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)(b * Hkv)), dim3(kSelThreads), lds, s, scores,
                     seq_len, P, max_pages, K, Hkv, heads, sel, sel_count);
  return hipGetLastError();
}

}  // namespace kvs
