// NF4 code table and fp32 decision thresholds (host, C++17).
//
// "QLoRA: How to fine-tune large language models with less memory", section
// "1. NormalFloat": sixteen 4-bit codes whose values follow a zero-centred
// normal distribution, denser near zero.  Construction used here (the
// NormalFloat layout the AQLoRA page calls bitsandbytes' NF4): with
// delta = 1 - (1/30 + 1/32)/2, eight positive values Phi^-1(p)/Phi^-1(delta)
// at the probabilities p = delta - j (delta - 1/2)/8, j = 0..7, seven negative
// values -Phi^-1(p)/Phi^-1(delta) at p = delta - j (delta - 1/2)/7, j = 0..6,
// and an exact zero; ascending, computed in double and rounded to float.
//
// Phi^-1 is solved here from Phi(x) = erfc(-x / sqrt 2) / 2 by bisection
// followed by Newton steps on std::erfc, to about 1e-15 relative; every table
// value lies far enough from an fp32 rounding boundary that this accuracy
// fixes its float exactly.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "nf4_host.hpp"

namespace nf4k {

static double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

static double normal_pdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

static double normal_quantile(double p) {
  double lo = -10.0, hi = 10.0;
  for (int i = 0; i < 80; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (normal_cdf(mid) < p) lo = mid;
    else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  for (int i = 0; i < 4; ++i) x -= (normal_cdf(x) - p) / normal_pdf(x);
  return x;
}

static NF4Consts build_consts() {
  const double delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
  const double z = normal_quantile(delta);
  double v[16];
  int n = 0;
  for (int j = 0; j <= 6; ++j) v[n++] = -normal_quantile(delta - j * (delta - 0.5) / 7.0) / z;
  v[n++] = 0.0;
  for (int j = 7; j >= 0; --j) v[n++] = normal_quantile(delta - j * (delta - 0.5) / 8.0) / z;
  // v is ascending by construction: negative side from -1 toward 0, then 0,
  // then the positive side from small to +1.
  NF4Consts c;
  for (int i = 0; i < 16; ++i) c.table[i] = (float)v[i];
  for (int j = 0; j < 15; ++j) {
    const double m = 0.5 * ((double)c.table[j] + (double)c.table[j + 1]);  // exact in double
    float t = (float)m;
    if ((double)t > m) t = std::nextafter(t, -INFINITY);
    c.thr[j] = t;
  }
  c.thr[15] = INFINITY;
  return c;
}

const NF4Consts& nf4_consts() {
  static const NF4Consts c = build_consts();
  return c;
}

static uint32_t bucket_of(float x) { return (uint32_t)std::fmaf(x, 16.0f, 16.0f); }

static NF4Enc build_enc() {
  const NF4Consts& c = nf4_consts();
  NF4Enc e;
  int owner[kBuckets];
  for (int k = 0; k < kBuckets; ++k) {
    e.bound[k] = INFINITY;
    owner[k] = -1;
  }
  const float margin = 1e-5f;
  for (int j = 0; j < 15; ++j) {
    const float t = c.thr[j];
    const uint32_t k = bucket_of(t);
    // one threshold per bucket, none near a bucket edge
    if (k >= (uint32_t)kBuckets || owner[k] >= 0) std::abort();
    if (bucket_of(t - margin) != k || bucket_of(t + margin) != k) std::abort();
    owner[k] = j;
    const float succ = std::nextafter(t, INFINITY);
    double u = 0.5 * ((double)t + (double)succ);  // exact: the rounding boundary above t
    if ((float)u == succ) u = std::nextafter(u, -INFINITY);  // a tie rounds up to succ: w on u counts
    e.bound[k] = u;
  }
  uint32_t below = 0;
  for (int k = 0; k < kBuckets; ++k) {
    e.base[k] = below;
    if (owner[k] >= 0) ++below;
    e.qlo[k] = c.table[e.base[k]];
    e.qhi[k] = c.table[owner[k] >= 0 ? e.base[k] + 1 : e.base[k]];
  }
  return e;
}

const NF4Enc& nf4_enc() {
  static const NF4Enc e = build_enc();
  return e;
}

}  // namespace nf4k
