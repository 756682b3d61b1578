// Host-visible constants of the NF4 format (no HIP dependency).
#pragma once

#include <stdint.h>

namespace nf4k {

// 4-bit codebooks: NF4 (the format of the QLoRA pages), the symmetric int4
// grid (c - 8) / 7, and the E2M1 4-bit float divided by 6 (-0 before +0).
enum { kCodebookNF4 = 0, kCodebookINT4 = 1, kCodebookFP4 = 2, kCodebooks = 3 };

// Code values of a codebook, ascending, passed by value to every kernel that
// decodes (the dequantized weight of code c is fl32(table[c] * scale)).
struct NF4Consts {
  float table[16];
  // thr[j]: the largest fp32 <= (table[j] + table[j+1]) / 2 (informational;
  // the encoders use NF4Enc)
  float thr[16];
};

// The tables, built once on first use (thread-safe static initialisation).
const NF4Consts& codebook_consts(int codebook);
inline const NF4Consts& nf4_consts() { return codebook_consts(kCodebookNF4); }

// Bucket table of the encoder.  The code of a weight w in a block with
// absmax m > 0 is the first nearest table value to x = fl32(w / m), i.e. the
// number of decision thresholds below x counted between distinct values.
//  * Bucket: k = trunc(fl32(bscale * x' + boffset)), bscale a power of two,
//    for any x' within 1e-5 of x (w times an approximate reciprocal of m).
//    Buckets are narrower than the smallest gap between two thresholds, so a
//    bucket holds at most one threshold, and no threshold lies within 1e-5
//    of a bucket edge, so x' and x see the same thresholds around the bucket.
//  * Inside the bucket the one threshold t is decided exactly without
//    dividing: fl32(w/m) > t  <=>  w/m is past the rounding boundary u between
//    t and its fp32 successor (or on it, when the tie rounds up), and u has 25
//    significant bits, so u*m is exact in fp64.  bound[k] is u (tie rounds
//    down) or the double just below u (tie rounds up; no fp32 w lies between
//    the two products), and x > t  <=>  fma(-bound[k], m, w) > 0 in fp64.
//    Buckets without a threshold have bound = +inf.
//  * code_lo[k] / code_hi[k]: the code below / above the bucket's threshold
//    (the first index of each distinct value), qlo / qhi their values.
// Thresholds below -1 are passed by every x; those at or above 1 by none.
constexpr int kMaxBuckets = 66;
struct NF4Enc {
  float bscale, boffset;
  int32_t nb;
  double bound[kMaxBuckets];
  uint32_t code_lo[kMaxBuckets];
  uint32_t code_hi[kMaxBuckets];
  float qlo[kMaxBuckets];
  float qhi[kMaxBuckets];
};
const NF4Enc& codebook_enc(int codebook);
inline const NF4Enc& nf4_enc() { return codebook_enc(kCodebookNF4); }

}  // namespace nf4k
