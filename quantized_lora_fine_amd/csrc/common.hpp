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
