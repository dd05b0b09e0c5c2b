// Bounded per-layer budgets of the ZigZagkv page (Eq. 4 and Eq. 6), host only.
//
//   u_l    = x_l / sum_l x_l                                   (Eq. 4)
//   beta_l = B_bound + (B - B_bound) * L * u_l                  (Eq. 6)
// Layers whose beta exceeds the context length n are pinned at n and Eq. 6 is
// applied again to the others with what is left of the total L * B (their
// shares renormalised), until no layer exceeds n.  Integer budgets take the
// floor of beta and hand the leftover units, one each, to the largest
// fractional parts (lower layer first on ties).
//
// Built with -ffp-contract=off: every product and sum is rounded on its own,
// in the order written, so results do not depend on FMA contraction.
#include <math.h>

#include <algorithm>
#include <vector>

#include "../../include/kvsel.h"

namespace kvsel {
void set_last_error(const char* msg);  // defined with the C ABI entry points
}

extern "C" kvsel_status kvsel_zigzag_budgets(const double* profile, int32_t L, int64_t n,
                                             int64_t avg_budget, int64_t floor_budget,
                                             int32_t* out) {
  auto bad = [](const char* msg) {
    kvsel::set_last_error(msg);
    return KVSEL_EINVAL;
  };
  kvsel::set_last_error("");
  if (!profile || !out) return bad("profile and out must be non-NULL");
  if (L < 1) return bad("L must be >= 1");
  if (n < 1 || n > 0x7fffffffLL) return bad("n must be in [1, 2^31)");
  if (floor_budget < 0 || floor_budget > avg_budget || avg_budget > n)
    return bad("need 0 <= floor_budget <= avg_budget <= n");
  for (int l = 0; l < L; ++l)
    if (!(profile[l] > 0.0) || !isfinite(profile[l])) return bad("profile entries must be finite and > 0");
  const long long total = (long long)L * avg_budget;
  if (total > 0x7fffffffLL) return bad("L * avg_budget overflows int32");

  double sx = 0.0;
  for (int l = 0; l < L; ++l) sx += profile[l];
  std::vector<double> u(L), beta(L, 0.0);
  for (int l = 0; l < L; ++l) u[l] = profile[l] / sx;  // Eq. 4

  std::vector<char> pinned(L, 0);
  int n_pinned = 0;
  for (;;) {
    const int n_free = L - n_pinned;
    const long long left = total - (long long)n_pinned * n;
    const long long spread = left - (long long)floor_budget * n_free;  // (B - B_bound) * L at first
    double su = 0.0;
    for (int l = 0; l < L; ++l)
      if (!pinned[l]) su += u[l];
    bool grew = false;
    for (int l = 0; l < L; ++l) {
      if (pinned[l]) continue;
      const double share = n_pinned == 0 ? u[l] : u[l] / su;
      beta[l] = (double)floor_budget + (double)spread * share;  // Eq. 6
    }
    for (int l = 0; l < L; ++l)
      if (!pinned[l] && beta[l] > (double)n) {
        pinned[l] = 1;
        ++n_pinned;
        grew = true;
      }
    if (!grew || n_pinned == L) break;
  }

  long long assigned = 0;
  std::vector<int> order;
  for (int l = 0; l < L; ++l) {
    long long v;
    if (pinned[l]) {
      v = n;
    } else {
      v = (long long)floor(beta[l]);
      order.push_back(l);
    }
    out[l] = (int32_t)v;
    assigned += v;
  }
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return (beta[a] - floor(beta[a])) > (beta[b] - floor(beta[b]));
  });
  long long leftover = total - assigned;
  for (size_t i = 0; leftover > 0 && !order.empty(); ++i) {
    const int l = order[i % order.size()];
    if (out[l] < n) {
      ++out[l];
      --leftover;
    }
    if (i > (size_t)4 * L + 8 && leftover > 0) break;  // cannot happen when total <= L * n
  }
  return KVSEL_OK;
}
