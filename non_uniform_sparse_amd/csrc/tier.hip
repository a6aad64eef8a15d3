// Host tier of stable heads (FlexiCache summary, tiered placement: a stable
// head keeps only its selected pages on the GPU and the rest in host memory,
// a rerank moves only the pages newly promoted into its selection; System
// engineering: GPU blocks freed and reused inside the rerank step, copies by
// a kernel that reads pinned host memory directly).
//
// offload_kernel, one wave per (head, page): after prefill, every resident
// page of a tiered head is copied to its host page host_base + p, 64 lanes
// moving 16 bytes each per load.
//
// promote_kernel, one 256-thread workgroup per (request, KV head), after the
// head's top-K.  In LDS: a bitmap of the selected pages, then the head's
// free slots (slot order) and the pages to promote (ascending page order).
//   1. Slots: a slot is kept when it holds a selected page that the table
//      maps to it; otherwise it is free, and the page it held goes back to
//      KVS_PAGE_ON_HOST (or -1 past the head's pages) if the table pointed
//      at this slot.
//   2. Pages: a selected page whose entry is KVS_PAGE_ON_HOST is promoted.
//   3. One block scan turns both flag sets into the two lists; promoted page
//      k goes into free slot k.  The copies run as one flat loop of 16-byte
//      chunks over all of the head's promoted pages, 8 loads from host
//      memory in flight per thread before their stores (reads over the host
//      link have microseconds of latency).
//   4. The table entries of the promoted pages and the slot records are
//      written last; the next kernel on the stream sees them.
// Writes in step 1 touch only unselected pages and step 2 reads only
// selected ones, so the two never meet.
#include "radix_select.h"
#include "kvs_launch.h"

namespace kvs {
namespace {

constexpr int P = 16;
constexpr int kPromoteThreads = kSelThreads;                 // 256
constexpr int kSlotsPerThread = kMaxSlots / kPromoteThreads;   // 4
constexpr int kBitmapWords = kMaxTierPages / 32;               // 256
constexpr int kPagesPerThread = kMaxTierPages / kPromoteThreads;
constexpr int kCopyDepth = 8;

__global__ __launch_bounds__(kPromoteThreads) void promote_kernel(CacheView c, HostTierView t,
                                                                  const int32_t* __restrict__ sel,
                                                                  const int32_t* __restrict__ sel_count,
                                                                  int K, HeadMask heads,
                                                                  int32_t* __restrict__ moved) {
  __shared__ uint32_t bm[kBitmapWords];
  __shared__ int s_free[kMaxSlots];
  __shared__ int s_prom[kMaxSlots];
  __shared__ int red[kSelWaves];
  __shared__ int totals[2];
  const int64_t rh = blockIdx.x;
  const int r = (int)(rh / c.Hkv), h = (int)(rh % c.Hkv);
  const int tid = threadIdx.x;
  const int64_t hb = t.host_base[rh];
  const int hs = c.head_slot[h];
  if (!heads.has(h) || hb < 0 || hs < 0 || hs >= c.Hkv) {   // uniform over the block
    if (moved && tid == 0) moved[rh] = 0;
    return;
  }
  int32_t* row = const_cast<int32_t*>(c.page_table) + ((int64_t)r * c.G + hs) * c.maxpg;
  const int npg = (clampi(c.seq_len[rh], 0, P * c.maxpg) + P - 1) / P;
  const int cnt = clampi(sel_count[rh], 0, K);
  int32_t* slot_page = t.slot_page + rh * t.slots;
  const int32_t* slot_phys = t.slot_phys + rh * t.slots;

  for (int w = tid; w < kBitmapWords; w += kPromoteThreads) bm[w] = 0u;
  __syncthreads();
  for (int i = tid; i < cnt; i += kPromoteThreads) {
    const int p = sel[rh * K + i];
    if (p >= 0 && p < npg) atomicOr(&bm[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  auto selected = [&](int p) { return (bm[p >> 5] >> (p & 31)) & 1u; };

  // 1. slots
  uint32_t free_bits = 0;
  int nfree = 0;
#pragma unroll
  for (int k = 0; k < kSlotsPerThread; ++k) {
    const int j = tid * kSlotsPerThread + k;
    if (j >= t.slots) break;
    const int ph = slot_phys[j];
    if (ph < 0 || ph >= c.num_pages) continue;   // unusable slot
    const int p = slot_page[j];
    const bool mapped = p >= 0 && p < c.maxpg && row[p] == ph;
    if (mapped && p < npg && selected(p)) continue;   // kept
    if (mapped) row[p] = p < npg ? KVS_PAGE_ON_HOST : -1;
    free_bits |= 1u << k;
    ++nfree;
  }
  // 2. pages to promote
  uint32_t prom_bits = 0;
  int nprom = 0;
  const int p_lo = tid * kPagesPerThread;
  for (int k = 0; k < kPagesPerThread; ++k) {
    const int p = p_lo + k;
    if (p >= npg) break;
    if (selected(p) && row[p] == KVS_PAGE_ON_HOST && hb + p < t.num_host_pages) {
      prom_bits |= 1u << k;
      ++nprom;
    }
  }
  // 3. lists, then the copies
  const int before = block_exclusive_scan((nfree << 16) | nprom, red);
  int fo = before >> 16, po = before & 0xffff;
  if (tid == kPromoteThreads - 1) {
    totals[0] = fo + nfree;
    totals[1] = po + nprom;
  }
#pragma unroll
  for (int k = 0; k < kSlotsPerThread; ++k)
    if ((free_bits >> k) & 1u) s_free[fo++] = tid * kSlotsPerThread + k;
  for (int k = 0; k < kPagesPerThread; ++k)
    if ((prom_bits >> k) & 1u) s_prom[po++] = p_lo + k;
  __syncthreads();
  const int total_free = totals[0];
  const int pairs = min(total_free, totals[1]);

  const int d = c.d;
  const int cpp_shift = d == 128 ? 9 : 10;   // 16-byte chunks per page: 2 P d * 2 / 16 = 4 d
  const int64_t page_elems = 2 * P * d;
  const uint16_t* host = static_cast<const uint16_t*>(t.host_kv);
  uint16_t* kv = static_cast<uint16_t*>(c.kv);
  const int chunks = pairs << cpp_shift;
  for (int base = 0; base < chunks; base += kPromoteThreads * kCopyDepth) {
    uint4 v[kCopyDepth];
#pragma unroll
    for (int u = 0; u < kCopyDepth; ++u) {
      const int i = base + u * kPromoteThreads + tid;
      if (i < chunks) {
        const int k = i >> cpp_shift, off = i & ((1 << cpp_shift) - 1);
        v[u] = ld16(host + (hb + s_prom[k]) * page_elems + 8 * off);
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyDepth; ++u) {
      const int i = base + u * kPromoteThreads + tid;
      if (i < chunks) {
        const int k = i >> cpp_shift, off = i & ((1 << cpp_shift) - 1);
        *reinterpret_cast<uint4*>(kv + (int64_t)slot_phys[s_free[k]] * page_elems + 8 * off) = v[u];
      }
    }
  }
  // 4. mappings
  for (int k = tid; k < total_free; k += kPromoteThreads) {
    const int j = s_free[k];
    if (k < pairs) {
      row[s_prom[k]] = slot_phys[j];
      slot_page[j] = s_prom[k];
    } else {
      slot_page[j] = -1;
    }
  }
  if (moved && tid == 0) moved[rh] = pairs;
}

template <int D>
__global__ __launch_bounds__(256) void offload_kernel(CacheView c, HostTierView t) {
  constexpr int CPL = 4 * D / 64;   // 16-byte chunks per lane of a page
  const int rh = blockIdx.y;
  const int r = rh / c.Hkv, h = rh % c.Hkv;
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t hb = t.host_base[rh];
  const int hs = c.head_slot[h];
  if (hb < 0 || hs < 0 || hs >= c.Hkv) return;
  const int npg = (clampi(c.seq_len[rh], 0, P * c.maxpg) + P - 1) / P;
  if (p >= npg || hb + p >= t.num_host_pages) return;
  const int phys = c.page_table[((int64_t)r * c.G + hs) * c.maxpg + p];
  if (phys < 0 || phys >= c.num_pages) return;
  const uint16_t* src = static_cast<const uint16_t*>(c.kv) + (int64_t)phys * 2 * P * D + 8 * lane;
  uint16_t* dst = static_cast<uint16_t*>(t.host_kv) + (hb + p) * 2 * P * D + 8 * lane;
  uint4 v[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) v[k] = ld16(src + 512 * k);
#pragma unroll
  for (int k = 0; k < CPL; ++k) *reinterpret_cast<uint4*>(dst + 512 * k) = v[k];
}

}  // namespace

hipError_t launch_promote(const CacheView& c, const HostTierView& t, const int32_t* sel,
                          const int32_t* sel_count, int K, const HeadMask& heads, int32_t* moved,
                          hipStream_t s) {
  hipLaunchKernelGGL(promote_kernel, dim3((unsigned)(c.b * c.Hkv)), dim3(kPromoteThreads), 0, s,
                     c, t, sel, sel_count, K, heads, moved);
  return hipGetLastError();
}

hipError_t launch_offload(const CacheView& c, const HostTierView& t, hipStream_t s) {
  const dim3 grid((unsigned)((c.maxpg + 3) / 4), (unsigned)(c.b * c.Hkv));
  if (c.d == 128)
    hipLaunchKernelGGL(offload_kernel<128>, grid, dim3(256), 0, s, c, t);
  else
    hipLaunchKernelGGL(offload_kernel<256>, grid, dim3(256), 0, s, c, t);
  return hipGetLastError();
}

}  // namespace kvs
