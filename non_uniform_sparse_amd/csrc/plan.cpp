// Host-side ahead-of-time planning (Tangram review, 3.2 Ragged Paging:
// budget-aware clustering; 3.3 AOT Load Balancing: the static split map).
// Pure C++; runs once per model / batch bucket, never on the decode step.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

#include "kvs_internal.h"
#include "kvs_launch.h"

namespace {

// round(min(B, cap) * 2^20), halves up.  B*2^20 < 2^21 and the scaling by a
// power of two is exact, so adding 1/2 and flooring is exact in double.
int64_t split_weight(double b, double cap) {
  if (cap > 0.0 && cap < b) b = cap;
  return (int64_t)std::floor(std::ldexp(b, 20) + 0.5);
}

bool valid_budget(double b) { return b > 0.0 && b <= 1.0; }

}  // namespace

extern "C" int kvs_cluster_heads(const double* budgets, int32_t L, int32_t Hkv, int32_t Hp,
                                 int32_t* head_slot) {
  using kvs::set_error;
  kvs::clear_error();
  if (!budgets || !head_slot) return set_error(KVS_EINVAL, "kvs_cluster_heads: null pointer");
  if (L < 1 || Hkv < 1 || Hp < 1 || Hkv % Hp)
    return set_error(KVS_EINVAL, "kvs_cluster_heads: need L >= 1, Hkv >= 1, Hkv %% Hp == 0");
  for (int64_t i = 0; i < (int64_t)L * Hkv; ++i)
    if (!valid_budget(budgets[i]))
      return set_error(KVS_EINVAL, "kvs_cluster_heads: budget %lld not in (0, 1]", (long long)i);
  std::vector<int32_t> order(Hkv);
  for (int32_t l = 0; l < L; ++l) {
    const double* row = budgets + (int64_t)l * Hkv;
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(),
                     [row](int32_t x, int32_t y) { return row[x] > row[y]; });
    for (int32_t pos = 0; pos < Hkv; ++pos) head_slot[(int64_t)l * Hkv + order[pos]] = pos;
  }
  return KVS_OK;
}

extern "C" int kvs_plan_split(const double* budgets, const int32_t* head_slot, int32_t L,
                              int32_t Hkv, int32_t Hp, double cap, int32_t T, int32_t* S) {
  using kvs::set_error;
  kvs::clear_error();
  if (!budgets || !head_slot || !S) return set_error(KVS_EINVAL, "kvs_plan_split: null pointer");
  if (L < 1 || Hkv < 1 || Hp < 1 || Hkv % Hp)
    return set_error(KVS_EINVAL, "kvs_plan_split: need L >= 1, Hkv >= 1, Hkv %% Hp == 0");
  const int32_t G = Hkv / Hp;
  if (T < G || T > kvs::kMaxSplitsPerRequest)
    return set_error(KVS_EINVAL, "kvs_plan_split: T=%d must lie in [G=%d, %d]", T, G,
                     kvs::kMaxSplitsPerRequest);
  if (std::isnan(cap)) return set_error(KVS_EINVAL, "kvs_plan_split: cap is NaN");
  std::vector<int64_t> phi(G);
  std::vector<char> seen(Hkv);
  for (int32_t l = 0; l < L; ++l) {
    std::fill(phi.begin(), phi.end(), 0);
    std::fill(seen.begin(), seen.end(), 0);
    for (int32_t h = 0; h < Hkv; ++h) {
      const double b = budgets[(int64_t)l * Hkv + h];
      const int32_t hs = head_slot[(int64_t)l * Hkv + h];
      if (!valid_budget(b))
        return set_error(KVS_EINVAL, "kvs_plan_split: budget [%d][%d] not in (0, 1]", l, h);
      if (hs < 0 || hs >= Hkv || seen[hs])
        return set_error(KVS_EINVAL, "kvs_plan_split: head_slot row %d is not a permutation", l);
      seen[hs] = 1;
      phi[hs / Hp] += split_weight(b, cap);
    }
    int32_t* row = S + (int64_t)l * G;
    for (int32_t i = 0; i < G; ++i) row[i] = 1;
    // Highest averages: each further split to the largest phi_i / S_i;
    // phi_i * S_b > phi_b * S_i compared exactly (both < 2^63), ties keep
    // the lower index.
    for (int32_t k = G; k < T; ++k) {
      int32_t best = 0;
      for (int32_t i = 1; i < G; ++i)
        if (phi[i] * row[best] > phi[best] * row[i]) best = i;
      ++row[best];
    }
  }
  return KVS_OK;
}
