// Host-visible constants of the NF4 format (no HIP dependency).
#pragma once

#include <stdint.h>

namespace nf4k {

// NF4 code values and the fp32 decision thresholds between neighbours,
// passed by value to every kernel that encodes or decodes.
struct NF4Consts {
  float table[16];
  // thr[j] is the largest fp32 <= (table[j] + table[j+1]) / 2, so that for
  // an fp32 x:  x > midpoint_j  <=>  x > thr[j].  A value exactly on a
  // midpoint is not greater than it and keeps the lower code.
  float thr[16];  // thr[15] is padding
};

// The table, built once on first use (thread-safe static initialisation).
const NF4Consts& nf4_consts();

// Bucket table of the encoder.  For an fp32 x in [-1, 1] the bucket is
// k = trunc(fl(16 x + 16)) in 0..32 (one rounding; 16 x is exact), a
// monotone function of x whose buckets are 1/16 wide, narrower than the
// smallest gap between two thresholds, so a bucket holds at most one
// threshold.  With base[k] = number of thresholds in buckets below k and
// thr[k] the threshold inside bucket k (+inf if none):
//   code(x) = #{j : x > thr_j} = base[k] + (x > thr[k]),
// and the dequantized value of that code is (x > thr[k]) ? qhi[k] : qlo[k].
constexpr int kBuckets = 33;
struct NF4Enc {
  float thr[kBuckets];
  uint32_t base[kBuckets];
  float qlo[kBuckets];
  float qhi[kBuckets];
};
const NF4Enc& nf4_enc();

}  // namespace nf4k
