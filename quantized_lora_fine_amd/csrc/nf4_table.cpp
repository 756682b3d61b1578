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

static void fill_thresholds(NF4Consts& c) {
  for (int j = 0; j < 15; ++j) {
    const double m = 0.5 * ((double)c.table[j] + (double)c.table[j + 1]);  // exact in double
    float t = (float)m;
    if ((double)t > m) t = std::nextafter(t, -INFINITY);
    c.thr[j] = t;
  }
  c.thr[15] = INFINITY;
}

static NF4Consts build_nf4() {
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
  fill_thresholds(c);
  return c;
}

// int4: code c -> (c - 8) / 7 (code 0 lies below -1 and is never chosen)
static NF4Consts build_int4() {
  NF4Consts c;
  for (int i = 0; i < 16; ++i) c.table[i] = (float)((double)(i - 8) / 7.0);
  fill_thresholds(c);
  return c;
}

// fp4: sign, 2 exponent bits, 1 mantissa bit (magnitudes 0 .5 1 1.5 2 3 4 6), divided by 6
static NF4Consts build_fp4() {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  NF4Consts c;
  for (int i = 0; i < 8; ++i) {
    c.table[7 - i] = (float)(-mag[i] / 6.0);
    c.table[8 + i] = (float)(mag[i] / 6.0);
  }
  c.table[7] = -0.0f;
  fill_thresholds(c);
  return c;
}

const NF4Consts& codebook_consts(int codebook) {
  static const NF4Consts t[kCodebooks] = {build_nf4(), build_int4(), build_fp4()};
  return t[codebook >= 0 && codebook < kCodebooks ? codebook : 0];
}

static uint32_t bucket_of(float x, float bscale, float boffset) {
  return (uint32_t)std::fmaf(x, bscale, boffset);
}

// Thresholds between distinct consecutive values; first index of each value.
struct Decisions {
  int n;
  float t[15];
  int lo[15], hi[15];  // code below / above threshold i
};

static Decisions decisions(const NF4Consts& c) {
  Decisions d;
  d.n = 0;
  int first = 0;  // first index of the current distinct value
  for (int j = 0; j < 15; ++j) {
    if (c.table[j + 1] == c.table[j]) continue;  // equal values: the lower code always wins
    const double m = 0.5 * ((double)c.table[j] + (double)c.table[j + 1]);
    float t = (float)m;
    if ((double)t > m) t = std::nextafter(t, -INFINITY);
    d.t[d.n] = t;
    d.lo[d.n] = first;
    d.hi[d.n] = j + 1;
    ++d.n;
    first = j + 1;
  }
  return d;
}

static bool try_grid(const Decisions& d, const NF4Consts& c, float bscale, float boffset, NF4Enc* e) {
  const int nb = (int)bucket_of(1.0f, bscale, boffset) + 1;
  if (nb > kMaxBuckets) return false;
  e->bscale = bscale;
  e->boffset = boffset;
  e->nb = nb;
  int owner[kMaxBuckets];
  for (int k = 0; k < nb; ++k) {
    owner[k] = -1;
    e->bound[k] = INFINITY;
  }
  const float margin = 1e-5f;
  int below_all = 0;
  for (int i = 0; i < d.n; ++i) {
    const float t = d.t[i];
    if (t < -1.0f - margin) {
      ++below_all;
      continue;
    }
    if (t >= 1.0f) continue;
    if (t < -1.0f + margin || t > 1.0f - margin) return false;
    const uint32_t k = bucket_of(t, bscale, boffset);
    if (k >= (uint32_t)nb || owner[k] >= 0) return false;
    if (bucket_of(t - margin, bscale, boffset) != k || bucket_of(t + margin, bscale, boffset) != k) return false;
    owner[k] = i;
    const float succ = std::nextafter(t, INFINITY);
    double u = 0.5 * ((double)t + (double)succ);  // exact: the rounding boundary above t
    if ((float)u == succ) u = std::nextafter(u, -INFINITY);  // a tie rounds up to succ: w on u counts
    e->bound[k] = u;
  }
  // reduced code (number of thresholds passed) -> table code
  int code_of[16];
  code_of[0] = d.n > 0 ? d.lo[0] : 0;
  for (int i = 0; i < d.n; ++i) code_of[i + 1] = d.hi[i];
  int passed = below_all;
  for (int k = 0; k < nb; ++k) {
    e->code_lo[k] = (uint32_t)code_of[passed];
    e->code_hi[k] = (uint32_t)code_of[owner[k] >= 0 ? passed + 1 : passed];
    if (owner[k] >= 0) ++passed;
    e->qlo[k] = c.table[e->code_lo[k]];
    e->qhi[k] = c.table[e->code_hi[k]];
  }
  return true;
}

static NF4Enc build_enc(int codebook) {
  const NF4Consts& c = codebook_consts(codebook);
  const Decisions d = decisions(c);
  static const float grids[4][2] = {{16.f, 16.f}, {16.f, 16.5f}, {32.f, 32.f}, {32.f, 32.5f}};
  NF4Enc e;
  for (const auto& g : grids)
    if (try_grid(d, c, g[0], g[1], &e)) return e;
  std::abort();  // no bucket grid separates the thresholds
}

const NF4Enc& codebook_enc(int codebook) {
  static const NF4Enc t[kCodebooks] = {build_enc(kCodebookNF4), build_enc(kCodebookINT4), build_enc(kCodebookFP4)};
  return t[codebook >= 0 && codebook < kCodebooks ? codebook : 0];
}

}  // namespace nf4k
