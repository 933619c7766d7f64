// Host-side activation-bit allocation of GAMP ("Closing the Null Space"
// explainer, methodology: allocation strategy) and the bit-operation count
// of a guided step (key contribution 4: report BOPs of the guided step, both
// branches). Declared in include/qlinear.h; no device work.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <numeric>
#include <vector>

#include "../../include/qlinear.h"

namespace ql {
ql_status set_error(ql_status st, const char* msg);  // qlinear_api.cpp
}

extern "C" ql_status qlinear_gamp_allocate(int32_t n_layers, const int64_t* macs,
                                           const double* gain, int32_t w_bits,
                                           int64_t budget_bops, int32_t* a_bits,
                                           int64_t* bops) {
  if (n_layers < 1) return ql::set_error(QL_ERR_ARG, "n_layers must be >= 1");
  if (!macs || !gain || !a_bits || !bops)
    return ql::set_error(QL_ERR_ARG, "macs, gain, a_bits or bops is NULL");
  if (w_bits != 4 && w_bits != 8) return ql::set_error(QL_ERR_ARG, "w_bits must be 4 or 8");
  // Promotion cost of layer l: macs * w_bits * (8 - 4) bit operations.
  std::vector<int64_t> cost(n_layers);
  int64_t total = 0;
  for (int32_t l = 0; l < n_layers; ++l) {
    if (macs[l] <= 0 || macs[l] > ((int64_t)1 << 52))
      return ql::set_error(QL_ERR_ARG, "macs must be in [1, 2^52]");
    if (!std::isfinite(gain[l]) || gain[l] < 0.0)
      return ql::set_error(QL_ERR_ARG, "gain must be finite and >= 0");
    cost[l] = macs[l] * w_bits * 4;
    total += cost[l];  // all layers at 4-bit activations
  }
  int64_t all8 = 0;  // the largest total the scan can reach
  for (int32_t l = 0; l < n_layers; ++l)
    if (__builtin_add_overflow(all8, 2 * cost[l], &all8))
      return ql::set_error(QL_ERR_ARG, "total BOPs overflow int64");
  if (budget_bops < total)
    return ql::set_error(QL_ERR_ARG, "budget is below the BOPs of all-4-bit activations");
  std::vector<double> ratio(n_layers);
  for (int32_t l = 0; l < n_layers; ++l) ratio[l] = gain[l] / (double)cost[l];
  std::vector<int32_t> order(n_layers);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return ratio[a] > ratio[b]; });
  std::vector<int32_t> out(n_layers, 4);
  for (int32_t l : order) {
    if (total + cost[l] <= budget_bops) {
      out[l] = 8;
      total += cost[l];
    }
  }
  std::copy(out.begin(), out.end(), a_bits);
  *bops = total;
  return ql::set_error(QL_OK, "");
}
