// GPU decoder of the KV-cache codec (CacheGen notes, 7: arithmetic decoding
// on the GPU with one thread per token's symbols; 3: anchors and deltas over
// groups of tokens).  The format is the one kvs.h states for
// kvs_codec_encode.
//
// One lane decodes one stream -- the symbols of one token over S channels --
// and a workgroup covers NG whole token groups of one (layer, K/V, channel
// slice), so every delta token finds its anchor in the same workgroup.
// Lanes are ordered anchors first: with groups of 10, wave 0 holds the 64
// anchors and waves 1-9 the 576 delta tokens, so a wave searches either the
// wide anchor tables (up to 256 symbols) or the narrow delta tables, never
// both.
//
// Channels go in blocks of up to 32.  Per block:
//   1. the block's 2 x 32 tables -- back to back in the table pool -- are
//      copied into LDS with their metadata and the channels' anchor ranges;
//   2. every lane decodes its block of symbols: r = range >> 16, the slice
//      index floor(code / r) (a float reciprocal, corrected to the exact
//      quotient), a binary search of the table in LDS, then at most two
//      byte renormalisations; symbols go to an LDS tile, 4 per dword (odd
//      row stride in dwords: no bank conflicts);
//   3. the tile is reconstructed -- an anchor lo + code*scale, a delta token
//      its anchor's value + q*bin, float32 product then sum, rounded once to
//      fp16 -- and written as 16-byte rows of 8 channels.
// Stream bytes are read a dword at a time with the next dword already in
// flight.  Every read is clamped into the buffers' stated lengths and every
// loop has a fixed bound, so a corrupt input decodes to garbage, never a
// fault or a hang.
#include <hip/hip_fp16.h>

#include "kvs_internal.h"
#include "kvs_launch.h"

namespace kvs {
namespace {

constexpr int kCB = 32;                    // channels per block
constexpr int kTabEntries = kCB * 2 * 256;  // LDS table capacity (entries)
constexpr int kMaxThreads = 1024;
constexpr int kRowDwords = kCB / 4 + 1;     // symbol tile row: 32 bytes + 4 pad

struct CodecArgs {
  const float* lo;
  const float* scale;
  const int32_t* tab_first;
  const int32_t* tab_n;
  const uint32_t* tab_off;
  const uint16_t* cdf;
  uint64_t cdf_len;
  const uint8_t* streams;
  const uint64_t* stream_off;
  uint64_t streams_len;
  uint16_t* out;
  int L, T, C, group, S, NG;
  float bins[3];
};

// Bytes of one stream, most significant first in a 64-bit buffer: `avail`
// bits are valid, and a dword is added whenever 32 or fewer remain (a symbol
// takes at most 16), with the dword after it already in flight.  Loads are
// unconditional, at an index clamped into the stream, so the compiler keeps
// the next dword in flight instead of waiting on a select; a valid stream
// never consumes what a clamped load returns (its decoder reads exactly the
// bytes its encoder wrote).
struct ByteReader {
  const uint32_t* base;
  uint32_t last;    // index of the stream's last dword
  uint32_t next;    // dword index of `nxt`
  uint32_t nxt;
  uint64_t bits;
  int avail;
  __device__ __forceinline__ uint32_t load(uint32_t i) const { return base[i < last ? i : last]; }
  __device__ __forceinline__ void refill() {
    if (avail <= 32) {
      bits |= (uint64_t)__builtin_bswap32(nxt) << (32 - avail);
      avail += 32;
      nxt = load(++next);
    }
  }
  // Starts a stream of ndw >= 1 dwords and returns the range decoder's first
  // code (bytes 1-4; byte 0 is the encoder's initial held byte).
  __device__ __forceinline__ uint32_t start(const uint32_t* p, uint32_t ndw) {
    base = p;
    last = ndw - 1;
    bits = ((uint64_t)__builtin_bswap32(load(0)) << 32) | __builtin_bswap32(load(1));
    nxt = load(2);
    next = 2;
    const uint32_t code = (uint32_t)(bits >> 24);
    bits <<= 40;
    avail = 24;
    refill();
    return code;
  }
};

__global__ __launch_bounds__(kMaxThreads) void codec_decode_kernel(CodecArgs a) {
  __shared__ uint16_t s_cdf[kTabEntries];
  // per table: LDS offset (bits 0-13), entries - 1 (14-21), first symbol + 128 (22-30)
  __shared__ uint32_t s_meta[2 * kCB];
  // per channel: binary-search steps of its anchor (bits 0-3) and delta (4-7) table
  __shared__ uint32_t s_steps[kCB];
  __shared__ float s_lo[kCB], s_scale[kCB];
  extern __shared__ uint32_t s_tile[];   // [NG * group rows][kRowDwords], sized at launch
  const int tid = threadIdx.x;
  const int g = a.group, NG = a.NG, TB = NG * g;
  const int lk = blockIdx.z;                  // l * 2 + kv
  const int l = lk >> 1;
  const int slice = blockIdx.y, NS = a.C / a.S;
  const int t0 = blockIdx.x * TB;
  // lane -> row of the workgroup's tokens: anchors first, then the deltas
  int row;
  if (tid < NG) {
    row = tid * g;
  } else {
    const int k = tid - NG;
    row = g > 1 ? (k / (g - 1)) * g + 1 + k % (g - 1) : TB;
  }
  const int t = t0 + row;
  const bool active = row < TB && t < a.T;
  const bool anchor = row % g == 0;
  const float bin = a.bins[(3 * l) / a.L];
  // which kinds of table this wave searches: its step count per channel is
  // the larger of those kinds' (uniform over the wave, a scalar loop)
  const bool wave_anchor = __ballot(active && anchor) != 0;
  const bool wave_delta = __ballot(active && !anchor) != 0;
  const int step_shift = wave_anchor && !wave_delta ? 0 : (!wave_anchor ? 4 : 8);

  uint32_t code = 0, rng = 0xffffffffu;
  ByteReader rd;
  rd.avail = 0;
  if (active) {
    const uint64_t s = ((uint64_t)lk * NS + slice) * (uint64_t)a.T + t;
    uint64_t b = a.stream_off[s] & ~(uint64_t)3, e = a.stream_off[s + 1] & ~(uint64_t)3;
    const uint64_t lim = a.streams_len & ~(uint64_t)3;
    b = b < lim ? b : lim;
    e = e < lim ? e : lim;
    if (e < b + 4) {   // not a stream (corrupt offsets): decode the buffer's first dword
      b = 0;
      e = 4;
    }
    code = rd.start(reinterpret_cast<const uint32_t*>(a.streams + b), (uint32_t)((e - b) >> 2));
  }

  const int64_t tab0 = (int64_t)lk * a.C * 2;
  for (int c0 = 0; c0 < a.S; c0 += kCB) {
    const int cb = min(kCB, a.S - c0);
    const int cg = slice * a.S + c0;            // first channel of the block
    // 1. tables, metadata and anchor ranges of the block
    const int64_t ti0 = tab0 + (int64_t)cg * 2;
    const uint64_t base = a.tab_off[ti0];
    if (tid < 2 * cb) {
      const int64_t ti = ti0 + tid;
      const int first = min(max(a.tab_first[ti], -128), 383);
      const int n = min(max(a.tab_n[ti], 1), 256);
      const uint64_t off = a.tab_off[ti];
      uint64_t lo = off >= base ? off - base : 0;
      lo = lo + n <= (uint64_t)kTabEntries ? lo : (uint64_t)(kTabEntries - n);
      s_meta[tid] = (uint32_t)lo | ((uint32_t)(n - 1) << 14) | ((uint32_t)(first + 128) << 22);
    }
    if (tid < cb) {
      const int n0 = min(max(a.tab_n[ti0 + 2 * tid], 1), 256) - 1;
      const int n1 = min(max(a.tab_n[ti0 + 2 * tid + 1], 1), 256) - 1;
      const uint32_t k0 = n0 ? 32 - __builtin_clz(n0) : 0, k1 = n1 ? 32 - __builtin_clz(n1) : 0;
      s_steps[tid] = k0 | (k1 << 4) | (max(k0, k1) << 8);
    }
    if (tid < cb) {
      s_lo[tid] = a.lo[(int64_t)lk * a.C + cg + tid];
      s_scale[tid] = a.scale[(int64_t)lk * a.C + cg + tid];
    }
    {
      const int64_t tl = ti0 + 2 * cb - 1;
      uint64_t end = (uint64_t)a.tab_off[tl] + (uint64_t)min(max(a.tab_n[tl], 1), 256);
      end = end < a.cdf_len ? end : a.cdf_len;
      const int cnt = end > base ? (int)min<uint64_t>(end - base, kTabEntries) : 0;
      for (int i = tid; i < cnt; i += blockDim.x) s_cdf[i] = a.cdf[base + i];
    }
    __syncthreads();
    // 2. decode
    if (active) {
      const int kind = anchor ? 0 : 1;
      uint32_t word = 0;
      for (int j = 0; j < cb; ++j) {
        const uint32_t meta = s_meta[2 * j + kind];
        const int lo_off = meta & 0x3fff, last = (meta >> 14) & 0xff;
        const int first = (int)(meta >> 22) - 128;
        // slice index floor(code / r): a float estimate, off by at most one,
        // corrected with the 32-bit remainder (|remainder| < 2 r <= 2^17)
        uint32_t r = rng >> 16;
        r = r ? r : 1u;
        uint32_t q = (uint32_t)((float)code * __builtin_amdgcn_rcpf((float)r));
        const uint32_t rem = code - q * r;
        q = (int32_t)rem < 0 ? q - 1 : (rem >= r ? q + 1 : q);
        const uint32_t v = q < 65535u ? q : 65535u;
        // largest x <= last with cdf[x] <= v (cdf[0] = 0): binary lifting over
        // the wave's step count, a compare and a select per step
        const int steps = __builtin_amdgcn_readfirstlane((s_steps[j] >> step_shift) & 0xf);
        int x = 0;
        for (int k = steps - 1; k >= 0; --k) {
          const int m = x + (1 << k);
          const uint32_t c = s_cdf[lo_off + min(m, last)];
          x = ((m <= last) & (c <= v)) ? m : x;
        }
        const uint32_t c_lo = s_cdf[lo_off + x];
        const uint32_t c_hi = x < last ? s_cdf[lo_off + x + 1] : 65536u;
        code -= r * c_lo;
        rng = r * (c_hi > c_lo ? c_hi - c_lo : 1u);
        // renormalise: 0, 1 or 2 bytes, branch-free
        const int nb = (rng < (1u << 24)) + (rng < (1u << 16));
        const uint32_t top = (uint32_t)(rd.bits >> 48);            // next two bytes
        code = (code << (8 * nb)) | (top >> (16 - 8 * nb));
        rng <<= 8 * nb;
        rd.bits <<= 8 * nb;
        rd.avail -= 8 * nb;
        rd.refill();
        word |= (uint32_t)((first + x) & 0xff) << (8 * (j & 3));
        if ((j & 3) == 3 || j == cb - 1) {
          s_tile[row * kRowDwords + (j >> 2)] = word;
          word = 0;
        }
      }
    }
    __syncthreads();
    // 3. reconstruct and store, 8 channels per item.  The product and the
    // sum are rounded separately, as the format states: contraction into a
    // fused multiply-add is off for the expressions of this loop.
    const int per_row = cb / 8;
    for (int it = tid; it < TB * per_row; it += blockDim.x) {
#pragma clang fp contract(off)
      const int rr = it / per_row, part = it % per_row;
      const int tt = t0 + rr;
      if (tt >= a.T) continue;
      const int ar = (rr / g) * g;
      const uint32_t* own = s_tile + rr * kRowDwords + 2 * part;
      const uint32_t* anc = s_tile + ar * kRowDwords + 2 * part;
      const uint32_t sw[2] = {own[0], own[1]}, aw[2] = {anc[0], anc[1]};
      uint32_t packed[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ch = 8 * part + e;
        const float code_a = (float)((aw[e >> 2] >> (8 * (e & 3))) & 0xffu);
        const float prod = code_a * s_scale[ch];
        float val = s_lo[ch] + prod;
        if (rr != ar) {
          const float dq = (float)(int8_t)((sw[e >> 2] >> (8 * (e & 3))) & 0xffu);
          const float step = dq * bin;
          val = val + step;
        }
        const uint32_t h = __half_as_ushort(__float2half_rn(val));
        if (e & 1) packed[e >> 1] |= h << 16; else packed[e >> 1] = h;
      }
      uint16_t* dst = a.out + (((int64_t)lk * a.T + tt) * a.C + cg + 8 * part);
      *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    }
    __syncthreads();
  }
}

}  // namespace

// Token groups per workgroup: at most 64 (or as many as 1024 threads hold),
// spread evenly over the workgroups a slice's T tokens need, so the last
// workgroup is not left mostly empty.
int codec_groups_per_block(int group, int T) {
  const int cap = group <= 16 ? 64 : kMaxThreads / group;
  const int groups = (T + group - 1) / group;
  const int blocks = (groups + cap - 1) / cap;
  return (groups + blocks - 1) / blocks;
}

hipError_t launch_codec_decode(const kvs_codec_layout& lay, const kvs_codec_chunk& ch, void* out,
                               hipStream_t s) {
  CodecArgs a;
  a.lo = ch.lo;
  a.scale = ch.scale;
  a.tab_first = ch.tab_first;
  a.tab_n = ch.tab_n;
  a.tab_off = ch.tab_off;
  a.cdf = ch.cdf;
  a.cdf_len = ch.cdf_len;
  a.streams = ch.streams;
  a.stream_off = ch.stream_off;
  a.streams_len = ch.streams_len;
  a.out = static_cast<uint16_t*>(out);
  a.L = lay.L;
  a.T = lay.T;
  a.C = lay.C;
  a.group = lay.group;
  a.S = lay.S;
  a.NG = codec_groups_per_block(lay.group, lay.T);
  for (int i = 0; i < 3; ++i) a.bins[i] = lay.bins[i];
  const int TB = a.NG * a.group;
  const int threads = (TB + 63) / 64 * 64;
  const dim3 grid((unsigned)((lay.T + TB - 1) / TB), (unsigned)(lay.C / lay.S),
                  (unsigned)(lay.L * 2));
  const size_t tile = (size_t)TB * kRowDwords * sizeof(uint32_t);
  hipLaunchKernelGGL(codec_decode_kernel, grid, dim3((unsigned)threads), tile, s, a);
  return hipGetLastError();
}

}  // namespace kvs
