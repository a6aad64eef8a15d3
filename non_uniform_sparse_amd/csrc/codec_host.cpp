// Host encoder of the KV-cache codec (CacheGen notes, 3: change-based
// encoding over groups of tokens, encoded offline; 7: 8-bit anchors, a delta
// bin per third of the layers, arithmetic coding with statistics per channel
// and layer).  The format is the one kvs.h states for kvs_codec_encode.
//
// Work is split over (layer, K/V) pairs, one host thread each at a time:
// quantize the pair's T x C values (IEEE float32, round half to even), count
// and normalise its 2 C tables, then range code its streams into a buffer of
// its own.  The pairs' tables and streams are then laid out in index order.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "kvs_internal.h"
#include "kvs_launch.h"

namespace kvs {
namespace {

constexpr uint32_t kTotal = 1u << 16;

// Exact fp16 -> float32.
float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  if (e == 0) {
    const float f = (float)m * 0x1p-24f;   // zero or subnormal, exact
    uint32_t b;
    memcpy(&b, &f, 4);
    b |= sign;
    float r;
    memcpy(&r, &b, 4);
    return r;
  }
  const uint32_t bits = e == 31 ? (sign | 0x7f800000u | (m << 13)) : (sign | ((e + 112) << 23) | (m << 13));
  float r;
  memcpy(&r, &bits, 4);
  return r;
}

// A byte-wise range coder over 32 bits: low carries into bit 32; the last
// byte produced is held back (`cache`) together with the 0xFF bytes after it
// (`pending` counts both) until a carry can no longer reach them.
struct RangeEncoder {
  std::vector<uint8_t>* out;
  uint64_t low = 0;
  uint32_t range = 0xffffffffu;
  uint8_t cache = 0;
  uint64_t pending = 1;

  void shift() {
    if (low < 0xff000000ull || low >= (1ull << 32)) {
      const uint8_t carry = (uint8_t)(low >> 32);
      out->push_back((uint8_t)(cache + carry));
      for (; pending > 1; --pending) out->push_back((uint8_t)(0xffu + carry));
      pending = 0;
      cache = (uint8_t)(low >> 24);
    }
    ++pending;
    low = (low & 0x00ffffffull) << 8;
  }
  void put(uint32_t cum, uint32_t freq) {
    const uint32_t r = range >> 16;
    low += (uint64_t)r * cum;
    range = r * freq;
    while (range < (1u << 24)) {
      range <<= 8;
      shift();
    }
  }
  void finish() {
    for (int i = 0; i < 5; ++i) shift();
  }
};

// A normalised table: symbols first .. first + n - 1, frequencies and
// cumulative frequencies.
struct Table {
  int first = 0;
  std::vector<uint32_t> freq, cum;
};

// Counts over symbols [base, base + counts.size()) -> normalised table.
Table make_table(const std::vector<uint64_t>& counts, int base) {
  Table t;
  uint64_t n = 0;
  int lo = -1, hi = -1;
  for (size_t i = 0; i < counts.size(); ++i) {
    if (!counts[i]) continue;
    n += counts[i];
    if (lo < 0) lo = (int)i;
    hi = (int)i;
  }
  if (n == 0) {
    t.first = 0;
    t.freq = {kTotal};
  } else {
    t.first = base + lo;
    t.freq.resize(hi - lo + 1);
    uint64_t sum = 0;
    for (int i = lo; i <= hi; ++i) {
      const uint64_t c = counts[i];
      const uint32_t f = c ? (uint32_t)std::max<uint64_t>(1, c * kTotal / n) : 0u;
      t.freq[i - lo] = f;
      sum += f;
    }
    size_t big = 0;
    for (size_t i = 1; i < t.freq.size(); ++i)
      if (t.freq[i] > t.freq[big]) big = i;
    t.freq[big] = (uint32_t)((int64_t)t.freq[big] + (int64_t)kTotal - (int64_t)sum);
  }
  t.cum.resize(t.freq.size());
  uint32_t c = 0;
  for (size_t i = 0; i < t.freq.size(); ++i) {
    t.cum[i] = c;
    c += t.freq[i];
  }
  return t;
}

// Everything one (layer, K/V) pair contributes.
struct PairOut {
  std::vector<float> lo, scale;          // [C]
  std::vector<Table> tables;             // [C][2]
  std::vector<uint8_t> bytes;            // its streams, in order
  std::vector<uint64_t> ends;            // end of each stream within bytes
};

void encode_pair(const kvs_codec_layout& lay, const uint16_t* x, int l, PairOut* o) {
  const int T = lay.T, C = lay.C, g = lay.group, S = lay.S;
  const float bin = lay.bins[(3 * l) / lay.L];
  std::vector<float> v((size_t)T * C);
  for (size_t i = 0; i < v.size(); ++i) v[i] = half_to_float(x[i]);
  o->lo.assign(C, 0.f);
  o->scale.assign(C, 0.f);
  for (int c = 0; c < C; ++c) {
    float lo = v[c], hi = v[c];
    for (int t = g; t < T; t += g) {
      const float a = v[(size_t)t * C + c];
      if (a < lo) lo = a;
      if (a > hi) hi = a;
    }
    o->lo[c] = lo;
    o->scale[c] = (hi - lo) / 255.0f;
  }
  std::vector<int16_t> sym((size_t)T * C);
  for (int t = 0; t < T; ++t) {
    const int ta = t - t % g;
    for (int c = 0; c < C; ++c) {
      const float val = v[(size_t)t * C + c];
      int s;
      if (t == ta) {
        const float sc = o->scale[c];
        s = sc > 0.f ? (int)std::min(255.f, std::max(0.f, rintf((val - o->lo[c]) / sc))) : 0;
      } else {
        const float d = rintf((val - v[(size_t)ta * C + c]) / bin);
        s = (int)std::min(127.f, std::max(-127.f, d));
      }
      sym[(size_t)t * C + c] = (int16_t)s;
    }
  }
  o->tables.resize((size_t)C * 2);
  std::vector<uint64_t> ca(256), cd(255);
  for (int c = 0; c < C; ++c) {
    std::fill(ca.begin(), ca.end(), 0);
    std::fill(cd.begin(), cd.end(), 0);
    for (int t = 0; t < T; ++t) {
      const int s = sym[(size_t)t * C + c];
      if (t % g == 0) ++ca[s]; else ++cd[s + 127];
    }
    o->tables[(size_t)c * 2] = make_table(ca, 0);
    o->tables[(size_t)c * 2 + 1] = make_table(cd, -127);
  }
  const int NS = C / S;
  o->ends.reserve((size_t)NS * T);
  for (int sl = 0; sl < NS; ++sl) {
    for (int t = 0; t < T; ++t) {
      RangeEncoder rc;
      rc.out = &o->bytes;
      const int kind = t % g == 0 ? 0 : 1;
      for (int c = sl * S; c < (sl + 1) * S; ++c) {
        const Table& tb = o->tables[(size_t)c * 2 + kind];
        const int i = sym[(size_t)t * C + c] - tb.first;
        rc.put(tb.cum[i], tb.freq[i]);
      }
      rc.finish();
      while (o->bytes.size() & 3) o->bytes.push_back(0);
      o->ends.push_back(o->bytes.size());
    }
  }
}

int check_layout(const kvs_codec_layout* p, const char* fn) {
  if (!p) return set_error(KVS_EINVAL, "%s: layout is NULL", fn);
  if (p->L < 1 || p->T < 1 || p->C < 8)
    return set_error(KVS_EINVAL, "%s: need L >= 1, T >= 1, C >= 8", fn);
  if (p->S < 8 || p->S % 8 || p->C % p->S)
    return set_error(KVS_EINVAL, "%s: S must be a multiple of 8 dividing C", fn);
  if (p->group < 1 || p->group > 320)
    return set_error(KVS_EINVAL, "%s: group %d not in [1, 320]", fn, p->group);
  for (int i = 0; i < 3; ++i)
    if (!(p->bins[i] > 0.f) || !std::isfinite(p->bins[i]))
      return set_error(KVS_EINVAL, "%s: bins must be positive and finite", fn);
  if ((int64_t)p->L * 2 * p->C * (256 + 255) >= ((int64_t)1 << 32) || (int64_t)p->T > (1 << 30) ||
      (int64_t)p->L * 2 > 65535 || p->C / p->S > 65535)
    return set_error(KVS_EUNSUPPORTED, "%s: chunk too large", fn);
  return KVS_OK;
}

}  // namespace

int codec_check_layout(const kvs_codec_layout* p, const char* fn) { return check_layout(p, fn); }

}  // namespace kvs

using namespace kvs;

extern "C" int kvs_codec_bounds(const kvs_codec_layout* layout, uint64_t* cdf_max,
                                uint64_t* streams_max) {
  clear_error();
  if (int rc = check_layout(layout, "kvs_codec_bounds")) return rc;
  if (!cdf_max || !streams_max) return set_error(KVS_EINVAL, "kvs_codec_bounds: null output");
  const uint64_t pairs = (uint64_t)layout->L * 2;
  const uint64_t S = layout->S;
  *cdf_max = pairs * layout->C * (256 + 255);
  // a symbol costs at most 16 bits plus 0.006 for the truncated r; one held
  // byte, four flushed, three of padding
  *streams_max = pairs * (layout->C / S) * layout->T * (2 * S + S / 512 + 12);
  return KVS_OK;
}

extern "C" int kvs_codec_encode(const kvs_codec_layout* layout, const uint16_t* x,
                                kvs_codec_chunk* out, int32_t threads) {
  clear_error();
  static const char* fn = "kvs_codec_encode";
  if (int rc = check_layout(layout, fn)) return rc;
  if (!x || !out || !out->lo || !out->scale || !out->tab_first || !out->tab_n || !out->tab_off ||
      !out->stream_off || (out->cdf_len && !out->cdf) || (out->streams_len && !out->streams))
    return set_error(KVS_EINVAL, "%s: null pointer", fn);
  const kvs_codec_layout lay = *layout;
  const int pairs = lay.L * 2;
  std::vector<PairOut> res(pairs);
  int nt = threads > 0 ? threads : (int)std::thread::hardware_concurrency();
  nt = std::max(1, std::min(nt, pairs));
  std::atomic<int> next{0};
  auto work = [&] {
    for (int p; (p = next.fetch_add(1)) < pairs;)
      encode_pair(lay, x + (size_t)p * lay.T * lay.C, p / 2, &res[p]);
  };
  std::vector<std::thread> pool;
  for (int i = 1; i < nt; ++i) pool.emplace_back(work);
  work();
  for (auto& th : pool) th.join();

  uint64_t cdf_need = 0, bytes_need = 0;
  for (const auto& r : res) {
    for (const auto& t : r.tables) cdf_need += t.freq.size();
    bytes_need += r.bytes.size();
  }
  if (out->cdf_len < cdf_need || out->streams_len < bytes_need) {
    out->cdf_len = cdf_need;
    out->streams_len = bytes_need;
    return set_error(KVS_ENOSPC, "%s: need %llu cdf entries and %llu stream bytes", fn,
                     (unsigned long long)cdf_need, (unsigned long long)bytes_need);
  }
  uint64_t ce = 0, be = 0, s = 0;
  out->stream_off[0] = 0;
  for (int p = 0; p < pairs; ++p) {
    const PairOut& r = res[p];
    for (int c = 0; c < lay.C; ++c) {
      out->lo[(size_t)p * lay.C + c] = r.lo[c];
      out->scale[(size_t)p * lay.C + c] = r.scale[c];
      for (int k = 0; k < 2; ++k) {
        const Table& t = r.tables[(size_t)c * 2 + k];
        const size_t i = ((size_t)p * lay.C + c) * 2 + k;
        out->tab_first[i] = t.first;
        out->tab_n[i] = (int32_t)t.freq.size();
        out->tab_off[i] = (uint32_t)ce;
        for (uint32_t v : t.cum) out->cdf[ce++] = (uint16_t)v;
      }
    }
    if (!r.bytes.empty()) memcpy(out->streams + be, r.bytes.data(), r.bytes.size());
    for (uint64_t e : r.ends) out->stream_off[++s] = be + e;
    be += r.bytes.size();
  }
  out->cdf_len = ce;
  out->streams_len = be;
  return KVS_OK;
}
