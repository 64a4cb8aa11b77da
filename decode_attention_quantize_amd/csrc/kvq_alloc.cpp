// kvq_alloc.cpp -- bit-width allocation across quantized components (host
// only): RateQuant technical summary (gist.science), methodology step 1
// (distortion-rate model D(b) = alpha beta^-b, weighted-distortion objective
// under a total bit budget, reverse water-filling) and step 3 (greedy
// integer widths, per-quantizer model calibration, keys and values as
// separate components).  The result feeds the per-layer (k_bits, v_bits)
// table of kvq_create; the fitting inputs come from the caller's own
// quantization-error measurements.
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/kvq.h"

extern "C" {

kvq_status kvq_fit_rate_distortion(int32_t n, const double* bits, const double* mse, double* alpha,
                                   double* beta) {
  if (n < 2 || !bits || !mse || !alpha || !beta) return KVQ_ERR_ARG;
  // least squares of ln mse against b: slope -ln beta, intercept ln alpha
  double sb = 0, sy = 0;
  for (int i = 0; i < n; ++i) {
    if (!(mse[i] > 0) || !std::isfinite(mse[i]) || !std::isfinite(bits[i])) return KVQ_ERR_ARG;
    sb += bits[i];
    sy += std::log(mse[i]);
  }
  const double mb = sb / n, my = sy / n;
  double sxx = 0, sxy = 0;
  for (int i = 0; i < n; ++i) {
    const double d = bits[i] - mb;
    sxx += d * d;
    sxy += d * (std::log(mse[i]) - my);
  }
  if (!(sxx > 0)) return KVQ_ERR_ARG;
  const double slope = sxy / sxx;
  *alpha = std::exp(my - slope * mb);
  *beta = std::exp(-slope);
  return KVQ_OK;
}

kvq_status kvq_waterfill_bits(int32_t n, const double* alpha, const double* beta, const double* w,
                              double total_bits, double* bits_out) {
  if (n < 1 || !alpha || !beta || !w || !bits_out || !std::isfinite(total_bits)) return KVQ_ERR_ARG;
  // every component's weighted marginal distortion w alpha ln(beta) beta^-b
  // equals one multiplier lambda; the budget fixes ln lambda
  std::vector<double> lnb(n), lc(n);
  double num = 0, den = 0;
  for (int i = 0; i < n; ++i) {
    if (!(alpha[i] > 0) || !(beta[i] > 1) || !(w[i] > 0)) return KVQ_ERR_ARG;
    lnb[i] = std::log(beta[i]);
    lc[i] = std::log(w[i]) + std::log(alpha[i]) + std::log(lnb[i]);
    num += lc[i] / lnb[i];
    den += 1.0 / lnb[i];
  }
  const double ln_lambda = (num - total_bits) / den;
  for (int i = 0; i < n; ++i) bits_out[i] = (lc[i] - ln_lambda) / lnb[i];
  return KVQ_OK;
}

kvq_status kvq_allocate_bits(int32_t n, const double* alpha, const double* beta, const double* w,
                             const int32_t* allowed, int32_t n_allowed, int32_t total_bits,
                             int32_t* bits_out) {
  if (n < 1 || !alpha || !beta || !w || !allowed || n_allowed < 1 || !bits_out) return KVQ_ERR_ARG;
  // the allowed widths, ascending and distinct
  std::vector<int32_t> lv;
  for (int k = 0; k < n_allowed; ++k) {
    if (allowed[k] < 1 || allowed[k] > 64) return KVQ_ERR_ARG;
    size_t p = 0;
    while (p < lv.size() && lv[p] < allowed[k]) ++p;
    if (p == lv.size() || lv[p] != allowed[k]) lv.insert(lv.begin() + static_cast<long>(p), allowed[k]);
  }
  for (int i = 0; i < n; ++i)
    if (!(alpha[i] > 0) || !(beta[i] > 1) || !(w[i] > 0)) return KVQ_ERR_ARG;
  int64_t left = static_cast<int64_t>(total_bits) - static_cast<int64_t>(n) * lv[0];
  if (left < 0) return KVQ_ERR_ARG;
  std::vector<int> level(n, 0);  // index into lv per component
  auto dist = [&](int i, int32_t b) { return w[i] * alpha[i] * std::pow(beta[i], -static_cast<double>(b)); };
  for (;;) {
    // the step with the largest weighted distortion reduction per bit that
    // still fits; ties to the lowest component index
    int best = -1;
    double best_gain = 0;
    for (int i = 0; i < n; ++i) {
      const int k = level[i];
      if (k + 1 >= static_cast<int>(lv.size())) continue;
      const int32_t step = lv[k + 1] - lv[k];
      if (step > left) continue;
      const double gain = (dist(i, lv[k]) - dist(i, lv[k + 1])) / step;
      if (best < 0 || gain > best_gain) {
        best = i;
        best_gain = gain;
      }
    }
    if (best < 0) break;
    left -= lv[level[best] + 1] - lv[level[best]];
    ++level[best];
  }
  for (int i = 0; i < n; ++i) bits_out[i] = lv[level[i]];
  return KVQ_OK;
}

}  // extern "C"
