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

// Bucket table of the encoder.  The code of a weight w in a block with
// absmax m > 0 is code(x) = #{j : x > thr_j} for x = fl32(w / m).
//  * Bucket: k = trunc(fl32(16 x' + 16)) in 0..32 for any x' within 1e-5 of
//    x (e.g. w times an approximate reciprocal of m).  Buckets are 1/16 wide,
//    narrower than the smallest gap between two thresholds, so a bucket holds
//    at most one threshold, and no threshold lies within 1e-5 of a bucket
//    edge, so x' and x see the same thresholds below and above the bucket.
//  * Inside the bucket the one threshold t is decided exactly without
//    dividing: fl32(w/m) > t  <=>  w/m is past the rounding boundary u between
//    t and its fp32 successor (or on it, when the tie rounds up), and u has 25
//    significant bits, so u*m is exact in fp64.  bound[k] is u (tie rounds
//    down) or the double just below u (tie rounds up; no fp32 w lies between
//    the two products), and x > t  <=>  fma(-bound[k], m, w) > 0 in fp64.
//    Buckets without a threshold have bound = +inf.
//  * base[k] = number of thresholds in buckets below k; the code is
//    base[k] + (x > t), and its value is qhi[k] or qlo[k].
constexpr int kBuckets = 33;
struct NF4Enc {
  double bound[kBuckets];
  uint32_t base[kBuckets];
  float qlo[kBuckets];
  float qhi[kBuckets];
};
const NF4Enc& nf4_enc();

}  // namespace nf4k
