// NF4 levels, built on the host when the library loads.
//
// Construction (QLoRA paper, Dettmers et al. 2023, "4-bit NormalFloat"): the
// levels are quantiles of the standard normal -- 8 on the positive side and 7
// on the negative side -- at probabilities spaced evenly between 1/2 and an
// offset delta = ((1 - 1/30) + (1 - 1/32)) / 2, plus one exact zero, divided
// by the largest magnitude so the book spans [-1, 1].  The quantile function
// here is our own: bisection on Phi(x) = erfc(-x / sqrt 2) / 2 to full double
// precision, polished by Newton steps; the result is rounded to fp32 once.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.h"

namespace ql {
namespace {

double phi_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double phi_pdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

double normal_quantile(double p) {
  double lo = -12.0, hi = 12.0;
  for (int it = 0; it < 200 && hi - lo > 0.0; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (phi_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  for (int it = 0; it < 2; ++it) x -= (phi_cdf(x) - p) / phi_pdf(x);
  return x;
}

Nf4Table build() {
  const double delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  double v[16];
  int n = 0;
  // positive side: 8 probabilities from delta down towards 1/2 (1/2 itself excluded)
  for (int i = 0; i < 8; ++i) v[n++] = normal_quantile(delta - i * (delta - 0.5) / 8.0);
  // negative side: 7 probabilities, mirrored
  for (int i = 0; i < 7; ++i) v[n++] = -normal_quantile(delta - i * (delta - 0.5) / 7.0);
  v[n++] = 0.0;
  std::sort(v, v + 16);
  double top = 0.0;
  for (double t : v) top = std::max(top, std::fabs(t));
  Nf4Table t{};
  for (int i = 0; i < 16; ++i) t.level[i] = (float)(v[i] / top);
  for (int i = 0; i < 15; ++i) {
    volatile float sum = t.level[i] + t.level[i + 1];   // one fp32 rounding
    t.mid[i] = sum * 0.5f;                               // exact halving
  }
  return t;
}

}  // namespace

const Nf4Table& nf4_table() {
  static Nf4Table table;
  static std::once_flag once;
  std::call_once(once, [] { table = build(); });
  return table;
}

}  // namespace ql
