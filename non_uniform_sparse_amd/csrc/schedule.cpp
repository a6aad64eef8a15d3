// Host-side schedules of the two "next" rows that decide, per head, how much
// work a call does: the Budget Reservation chunk quota of a chunked prefill
// (Tangram review, 3.1) and the stability-aware rerank schedule of decoding
// over steps (FlexiCache summary, Method: stable heads reuse their page
// selection between periodic reranks).  Pure C++, integer-exact.
#include <stdint.h>

#include <cmath>

#include "kvs_internal.h"
#include "kvs_launch.h"

namespace {

// ceil(B * x) on the exact binary value of B (0 < B <= 1), x >= 0.  B is
// m * 2^e with m a 53-bit integer, so B * x = (m * x) * 2^e with m * x <
// 2^85 held exactly in 128 bits, and the ceiling of a scaling by 2^e (e < 0)
// is a shift of (m * x + 2^-e - 1).
int64_t kept_after(double B, int64_t x) {
  if (x <= 0) return 0;
  int ex = 0;
  const double f = std::frexp(B, &ex);                      // B = f * 2^ex, f in [0.5, 1)
  const int64_t m = (int64_t)std::ldexp(f, 53);             // exact
  const int e = ex - 53;                                    // B = m * 2^e
  const unsigned __int128 mx = (unsigned __int128)m * (unsigned __int128)x;
  if (e >= 0) return (int64_t)(mx << e);                    // not reached for B <= 1
  const int k = -e;
  if (k >= 127) return mx > 0 ? 1 : 0;                      // 0 < B*x < 1
  const unsigned __int128 one = 1;
  return (int64_t)((mx + (one << k) - 1) >> k);
}

}  // namespace

extern "C" int kvs_prefill_quota(const double* budgets, const int64_t* contexts, int32_t b,
                                 int32_t Hkv, int64_t start, int32_t chunk, int32_t* quota) {
  using kvs::set_error;
  kvs::clear_error();
  const char* fn = "kvs_prefill_quota";
  if (!budgets || !contexts || !quota) return set_error(KVS_EINVAL, "%s: null pointer", fn);
  if (b < 1 || Hkv < 1) return set_error(KVS_EINVAL, "%s: need b >= 1 and Hkv >= 1", fn);
  if (start < 0 || chunk < 1 || start > ((int64_t)1 << 40))
    return set_error(KVS_EINVAL, "%s: need 0 <= start <= 2^40 and chunk >= 1", fn);
  for (int32_t h = 0; h < Hkv; ++h)
    if (!(budgets[h] > 0.0 && budgets[h] <= 1.0))
      return set_error(KVS_EINVAL, "%s: budget %d not in (0, 1]", fn, h);
  for (int32_t r = 0; r < b; ++r)
    if (contexts[r] < 1 || contexts[r] > ((int64_t)1 << 40))
      return set_error(KVS_EINVAL, "%s: context %d not in [1, 2^40]", fn, r);
  const int64_t end = start + chunk;
  for (int32_t r = 0; r < b; ++r) {
    const int64_t N = contexts[r];
    const int64_t a = start < N ? start : N, e = end < N ? end : N;
    for (int32_t h = 0; h < Hkv; ++h)
      quota[(int64_t)r * Hkv + h] = (int32_t)(kept_after(budgets[h], e) - kept_after(budgets[h], a));
  }
  return KVS_OK;
}

extern "C" int kvs_rerank_heads(const uint8_t* stable, int32_t Hkv, int32_t step, int32_t period,
                                uint8_t* due) {
  using kvs::set_error;
  kvs::clear_error();
  const char* fn = "kvs_rerank_heads";
  if (!stable || !due) return set_error(KVS_EINVAL, "%s: null pointer", fn);
  if (Hkv < 1 || step < 0 || period < 1)
    return set_error(KVS_EINVAL, "%s: need Hkv >= 1, step >= 0 and period >= 1", fn);
  const bool all = step % period == 0;
  for (int32_t h = 0; h < Hkv; ++h) due[h] = (uint8_t)(all || !stable[h]);
  return KVS_OK;
}
