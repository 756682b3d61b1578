// MFMA-only probe (gfx950): the bf16 matrix-core rate this chip sustains with
// no memory traffic and no LDS, the ceiling the fused GEMM's MFMA work is
// measured against besides the dense peak.  Every wave issues back-to-back
// v_mfma_f32_32x32x16_bf16 on eight independent accumulators (the consumer
// wave shape of the fused GEMM: eight 32x32 tiles), with operands that hold
// pseudo-random bf16 values (random operands draw more power than constant
// ones, and the clock follows power).  Not part of the layer.
#include "common.hpp"
#include "launch.hpp"

namespace nf4k {

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// a bf16 pair of magnitude in [0.5, 2) with random sign and mantissa bits
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t seed) {
  const uint32_t r = mix32(seed);
  const uint32_t lo = 0x3F00u | (r & 0x807Fu) | ((r >> 7) & 0x0080u);
  const uint32_t hi = 0x3F00u | ((r >> 16) & 0x807Fu) | ((r >> 23) & 0x0080u);
  return lo | (hi << 16);
}

__global__ __launch_bounds__(512) void k_mfma_peak(int iters, float* __restrict__ out) {
  const uint32_t gid = blockIdx.x * 512u + threadIdx.x;
  bf16x8 a[2], b[8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = rand_bf16x2(gid * 64u + 8u * j + e);
    a[j] = __builtin_bit_cast(bf16x8, v);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = rand_bf16x2(gid * 64u + 16u + 4u * j + e);
    b[j] = __builtin_bit_cast(bf16x8, v);
  }
  floatx16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  // two rounds per trip, one with each A operand (iters is rounded up to even)
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[0], acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[1], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[j][v];
  out[gid] = s;
}

hipError_t launch_mfma_peak(int iters, int workgroups, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_mfma_peak, dim3((unsigned)workgroups), dim3(512), 0, st, iters, out);
  return hipGetLastError();
}

}  // namespace nf4k
