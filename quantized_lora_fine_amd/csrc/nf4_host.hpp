// Host-visible constants of the NF4 format (no HIP dependency).
#pragma once

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

}  // namespace nf4k
