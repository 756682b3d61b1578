// NF4 quantize / dequantize / reconstruction-error / top-K kernels (gfx950).
//
// The weight is a row-major fp32 [rows][cols] array with cols % 64 == 0, so
// block b is the 64 consecutive floats starting at element 64*b and no block
// crosses a row.  One workgroup (256 threads, 4 wave64s) owns one group of 256
// consecutive blocks (16,384 weights): each wave streams 64 blocks in 16
// rounds; in a round the 16 lanes of a DPP row read one block as 16 x float4
// (the wave reads 1 KiB contiguous), so loads are fully coalesced, the block
// absmax is a 4-step DPP max inside the row, and the double-quantization
// group max needs no second pass over HBM.
//
// Format ("QLoRA: How to fine-tune large language models with less memory",
// sections "1. NormalFloat" and "2. Double quantization"): 4-bit codes, two
// per byte (even element in the low nibble), one fp32 absmax per 64 weights,
// or one 8-bit scale code per block plus an fp32 step per 256 blocks.
#include "common.hpp"
#include "launch.hpp"

namespace nf4k {

// ---------------------------------------------------------------------------
// quantize
// ---------------------------------------------------------------------------
template <bool DQ>
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ W, int64_t nblocks,
                                                  uint8_t* __restrict__ codes,
                                                  float* __restrict__ absmax,
                                                  uint8_t* __restrict__ c8,
                                                  float* __restrict__ dqs, NF4Consts cst) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane >> 4;   // block slot within a round (DPP row)
  const int l16 = lane & 15;   // lane within the row: elements 4*l16 .. 4*l16+3
  const int64_t g = blockIdx.x;
  const int64_t b0 = g * 256 + wave * 64;

  floatx4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t blk = b0 + i * 4 + sub;
    if (blk < nblocks) {
      v[i] = __builtin_nontemporal_load((const floatx4*)(W + blk * 64 + l16 * 4));
    } else {
      v[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }

  float amax[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float m = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
    m = row16_max(m);
    amax[i] = m;
    uint32_t p;
    if (m > 0.f) {
      p = nf4_encode(v[i].x / m, cst) | (nf4_encode(v[i].y / m, cst) << 4) |
          (nf4_encode(v[i].z / m, cst) << 8) | (nf4_encode(v[i].w / m, cst) << 12);
    } else {
      p = 0x7777u;  // all-zero block: every element takes the exact-zero code
    }
    const int64_t blk = b0 + i * 4 + sub;
    if (blk < nblocks) *(uint16_t*)(codes + blk * 32 + l16 * 2) = (uint16_t)p;
  }

  // lane l16 of row `sub` owns the block of round l16: blk = b0 + 4*l16 + sub
  float mine = amax[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mine = (l16 == i) ? amax[i] : mine;
  const int64_t myblk = b0 + l16 * 4 + sub;

  if constexpr (!DQ) {
    if (myblk < nblocks) absmax[myblk] = mine;
  } else {
    __shared__ float red[4];
    float gm = mine;
    gm = fmaxf(gm, __shfl_xor(gm, 1));
    gm = fmaxf(gm, __shfl_xor(gm, 2));
    gm = fmaxf(gm, __shfl_xor(gm, 4));
    gm = fmaxf(gm, __shfl_xor(gm, 8));
    gm = fmaxf(gm, __shfl_xor(gm, 16));
    gm = fmaxf(gm, __shfl_xor(gm, 32));
    if (lane == 0) red[wave] = gm;
    __syncthreads();
    gm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float S = gm / 255.0f;
    if (tid == 0) dqs[g] = S;
    if (myblk < nblocks) {
      uint8_t q = 0;
      if (S > 0.f) q = (uint8_t)fminf(255.f, rintf(mine / S));
      c8[myblk] = q;
    }
  }
}

// ---------------------------------------------------------------------------
// dequantize: each thread expands one code dword (8 weights of one block)
// ---------------------------------------------------------------------------
template <bool DQ, bool BF16>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes,
                                                    const void* __restrict__ absmax,
                                                    const float* __restrict__ dqs,
                                                    int64_t nwords, void* __restrict__ out,
                                                    NF4Consts cst) {
  __shared__ float tab[16];
  if (threadIdx.x < 16) tab[threadIdx.x] = cst.table[threadIdx.x];
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nwords; t += stride) {
    const uint32_t w = __builtin_nontemporal_load((const uint32_t*)codes + t);
    const int64_t blk = t >> 3;
    float sc;
    if constexpr (DQ) {
      sc = (float)((const uint8_t*)absmax)[blk] * dqs[blk >> 8];
    } else {
      sc = ((const float*)absmax)[blk];
    }
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = tab[(w >> (4 * e)) & 15u] * sc;
    if constexpr (BF16) {
      const u32x4 o = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                       pack_bf16x2(f[6], f[7])};
      __builtin_nontemporal_store(o, (u32x4*)out + t);
    } else {
      floatx4* o = (floatx4*)out + 2 * t;
      __builtin_nontemporal_store((floatx4{f[0], f[1], f[2], f[3]}), o);
      __builtin_nontemporal_store((floatx4{f[4], f[5], f[6], f[7]}), o + 1);
    }
  }
}

// ---------------------------------------------------------------------------
// reconstruction error, stage 1: per-group fp64 partial sums of (w - w_hat)^2
// and w^2 (encode/decode in fp32 as the format defines, differences and
// squares in fp64).  Same block/group mapping as k_quantize; the weights stay in
// registers between the absmax, group-max and encode/decode steps.
// ---------------------------------------------------------------------------
template <bool DQ>
__global__ __launch_bounds__(256) void k_error_partial(const float* __restrict__ W, int64_t nblocks,
                                                       double* __restrict__ part, NF4Consts cst) {
  __shared__ float tab[16];
  __shared__ float redf[4];
  __shared__ double redd[2][4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane >> 4;
  const int l16 = lane & 15;
  const int64_t g = blockIdx.x;
  const int64_t b0 = g * 256 + wave * 64;
  if (tid < 16) tab[tid] = cst.table[tid];

  floatx4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t blk = b0 + i * 4 + sub;
    if (blk < nblocks) {
      v[i] = __builtin_nontemporal_load((const floatx4*)(W + blk * 64 + l16 * 4));
    } else {
      v[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float amax[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float m = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
    amax[i] = row16_max(m);
  }
  float S = 0.f;
  if constexpr (DQ) {
    float gm = amax[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) gm = fmaxf(gm, amax[i]);
    gm = fmaxf(gm, __shfl_xor(gm, 16));
    gm = fmaxf(gm, __shfl_xor(gm, 32));
    if (lane == 0) redf[wave] = gm;
  }
  __syncthreads();  // also publishes tab[]
  if constexpr (DQ) {
    const float gm = fmaxf(fmaxf(redf[0], redf[1]), fmaxf(redf[2], redf[3]));
    S = gm / 255.0f;
  }

  double dsum = 0.0, wsum = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float m = amax[i];
    float sc = m;
    if constexpr (DQ) sc = (S > 0.f) ? fminf(255.f, rintf(m / S)) * S : 0.f;
    const float w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t c = (m > 0.f) ? nf4_encode(w4[e] / m, cst) : 7u;
      const float wh = tab[c] * sc;
      // fp64 from here on: squares of fp32 weights can leave the fp32 range
      const double wd = (double)w4[e];
      const double d = wd - (double)wh;
      dsum = fma(d, d, dsum);
      wsum = fma(wd, wd, wsum);
    }
  }
  // fixed-order reduction: xor tree inside the wave, then waves 0..3 in order
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    dsum += __shfl_xor(dsum, o);
    wsum += __shfl_xor(wsum, o);
  }
  if (lane == 0) {
    redd[0][wave] = dsum;
    redd[1][wave] = wsum;
  }
  __syncthreads();
  if (tid == 0) {
    part[2 * g + 0] = ((redd[0][0] + redd[0][1]) + redd[0][2]) + redd[0][3];
    part[2 * g + 1] = ((redd[1][0] + redd[1][1]) + redd[1][2]) + redd[1][3];
  }
}

// stage 2: one workgroup sums the per-group partials in a fixed order.
__global__ __launch_bounds__(256) void k_error_final(const double* __restrict__ part, int64_t ngroups,
                                                     double* __restrict__ err) {
  __shared__ double sd[256], sw[256];
  const int tid = threadIdx.x;
  double d = 0.0, w = 0.0;
  for (int64_t g = tid; g < ngroups; g += 256) {
    d += part[2 * g];
    w += part[2 * g + 1];
  }
  sd[tid] = d;
  sw[tid] = w;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      sd[tid] += sd[tid + s];
      sw[tid] += sw[tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) err[0] = (sw[0] > 0.0) ? sqrt(sd[0]) / sqrt(sw[0]) : 0.0;
}

// ---------------------------------------------------------------------------
// top-K by rank counting: rank(i) = #{j : e_j > e_i or (e_j == e_i and j < i)}
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_topk(const double* __restrict__ e, int n, int k,
                                               int* __restrict__ idx) {
  __shared__ double tile[1024];
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const double ei = (i < n) ? e[i] : 0.0;
    int rank = 0;
    for (int t0 = 0; t0 < n; t0 += 1024) {
      __syncthreads();
      if (t0 + (int)threadIdx.x < n) tile[threadIdx.x] = e[t0 + threadIdx.x];
      __syncthreads();
      const int lim = min(1024, n - t0);
      for (int jj = 0; jj < lim; ++jj) {
        const double ej = tile[jj];
        const int j = t0 + jj;
        rank += (ej > ei || (ej == ei && j < i)) ? 1 : 0;
      }
    }
    if (i < n && rank < k) idx[rank] = i;
  }
}

// ---------------------------------------------------------------------------
// host-side launchers (called from the C ABI layer)
// ---------------------------------------------------------------------------
hipError_t launch_quantize(const float* W, int64_t nblocks, bool dq, uint8_t* codes, void* absmax,
                           float* dqs, const NF4Consts& c, hipStream_t st) {
  const int64_t ng = (nblocks + 255) / 256;
  if (ng == 0) return hipSuccess;
  if (dq) {
    hipLaunchKernelGGL(k_quantize<true>, dim3((unsigned)ng), dim3(256), 0, st, W, nblocks, codes,
                       nullptr, (uint8_t*)absmax, dqs, c);
  } else {
    hipLaunchKernelGGL(k_quantize<false>, dim3((unsigned)ng), dim3(256), 0, st, W, nblocks, codes,
                       (float*)absmax, nullptr, nullptr, c);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const void* absmax, const float* dqs, int64_t nweights,
                             bool dq, bool bf16, void* out, const NF4Consts& c, hipStream_t st) {
  const int64_t nwords = nweights / 8;
  if (nwords == 0) return hipSuccess;
  int64_t blocks = (nwords + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  const dim3 gr((unsigned)blocks), bl(256);
  if (dq && bf16) hipLaunchKernelGGL((k_dequantize<true, true>), gr, bl, 0, st, codes, absmax, dqs, nwords, out, c);
  if (dq && !bf16) hipLaunchKernelGGL((k_dequantize<true, false>), gr, bl, 0, st, codes, absmax, dqs, nwords, out, c);
  if (!dq && bf16) hipLaunchKernelGGL((k_dequantize<false, true>), gr, bl, 0, st, codes, absmax, dqs, nwords, out, c);
  if (!dq && !bf16) hipLaunchKernelGGL((k_dequantize<false, false>), gr, bl, 0, st, codes, absmax, dqs, nwords, out, c);
  return hipGetLastError();
}

hipError_t launch_error(const float* W, int64_t nblocks, bool dq, double* part, double* err,
                        const NF4Consts& c, hipStream_t st) {
  const int64_t ng = (nblocks + 255) / 256;
  if (ng > 0) {
    if (dq) {
      hipLaunchKernelGGL(k_error_partial<true>, dim3((unsigned)ng), dim3(256), 0, st, W, nblocks, part, c);
    } else {
      hipLaunchKernelGGL(k_error_partial<false>, dim3((unsigned)ng), dim3(256), 0, st, W, nblocks, part, c);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_error_final, dim3(1), dim3(256), 0, st, part, ng, err);
  return hipGetLastError();
}

hipError_t launch_topk(const double* e, int n, int k, int* idx, hipStream_t st) {
  if (k == 0 || n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk, dim3(1), dim3(1024), 0, st, e, n, k, idx);
  return hipGetLastError();
}

}  // namespace nf4k
