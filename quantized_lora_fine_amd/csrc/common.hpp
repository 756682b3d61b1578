// Device helpers shared by the libnf4lora kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_host.hpp"

namespace nf4k {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// Nearest code of an fp32 x in [-1, 1]: the number of thresholds below x,
// found by a 4-level binary search over the 15 ordered thresholds.
__device__ __forceinline__ uint32_t nf4_encode(float x, const NF4Consts& c) {
  const bool b3 = x > c.thr[7];
  const float t2 = b3 ? c.thr[11] : c.thr[3];
  const bool b2 = x > t2;
  const float t1 = b3 ? (b2 ? c.thr[13] : c.thr[9]) : (b2 ? c.thr[5] : c.thr[1]);
  const bool b1 = x > t1;
  float t0;
  if (b3) {
    t0 = b2 ? (b1 ? c.thr[14] : c.thr[12]) : (b1 ? c.thr[10] : c.thr[8]);
  } else {
    t0 = b2 ? (b1 ? c.thr[6] : c.thr[4]) : (b1 ? c.thr[2] : c.thr[0]);
  }
  const bool b0 = x > t0;
  return (uint32_t)b3 * 8u + (uint32_t)b2 * 4u + (uint32_t)b1 * 2u + (uint32_t)b0;
}

// Max over the 16 lanes of a DPP row (lanes 16k .. 16k+15); every lane of the
// row receives the result.
__device__ __forceinline__ float row16_max(float v) {
  int x = __builtin_bit_cast(int, v);
  // quad_perm [1,0,3,2] and [2,3,0,1]: max over each quad
  x = __builtin_bit_cast(int, fmaxf(__builtin_bit_cast(float, x),
      __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false))));
  x = __builtin_bit_cast(int, fmaxf(__builtin_bit_cast(float, x),
      __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false))));
  // row_half_mirror: lane i <-> 7-i inside each 8 -> max over 8
  x = __builtin_bit_cast(int, fmaxf(__builtin_bit_cast(float, x),
      __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false))));
  // row_mirror: lane i <-> 15-i inside each 16 -> max over 16
  x = __builtin_bit_cast(int, fmaxf(__builtin_bit_cast(float, x),
      __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false))));
  return __builtin_bit_cast(float, x);
}

// Sum over the 16 lanes of a DPP row, same pattern as row16_max (fixed order,
// identical result in every lane of the row).
__device__ __forceinline__ double row16_sum(double v) {
  double s = v;
  s += __shfl_xor(s, 1, 16);
  s += __shfl_xor(s, 2, 16);
  s += __shfl_xor(s, 4, 16);
  s += __shfl_xor(s, 8, 16);
  return s;
}

}  // namespace nf4k
