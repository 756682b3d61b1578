// Rank-r adapter products of the QLoRA linear (gfx950).
//
// With X [M][h], dY [M][o], L1 [h][r], L2 [r][o] (bf16) the adapter path of
// equation (3) ("QLoRA: How to fine-tune large language models with less
// memory", "The algebra" section) and its backward need four skinny
// products with one dimension equal to the rank r:
//   T   = X L1            [M][r]   (forward; saved for the backward)
//   G   = s dY L2^T       [M][r]   (backward)
//   dL2 = s T^T dY        [r][o]   (backward, contraction over tokens)
//   dL1 = X^T G           [h][r]   (backward, contraction over tokens)
// All four stream a big [M][*] bf16 operand once from HBM against a small
// operand that stays in L2/LDS, on bf16 MFMA with fp32 accumulation.  The
// long contraction is split over workgroups; each split writes an fp32
// partial and a second kernel adds the partials in a fixed order, so results
// do not depend on scheduling (no floating-point atomics).
//
// Internally r is padded to RP = 16*ceil(r/16); padded rows/columns are zero.
#include "common.hpp"
#include "launch.hpp"

namespace nf4k {

// ---------------------------------------------------------------------------
// layout prep: out[i][j] = (i < irows && j < jcols) ? in[i*si + j*sj] : 0
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pad_transpose(const uint16_t* __restrict__ in, int64_t si, int64_t sj,
                                                       int64_t irows, int64_t jcols, uint16_t* __restrict__ out,
                                                       int64_t orows, int64_t ocols) {
  const int64_t total = orows * ocols;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t i = t / ocols;
    const int64_t j = t - i * ocols;
    out[t] = (i < irows && j < jcols) ? in[i * si + j * sj] : (uint16_t)0;
  }
}

// ---------------------------------------------------------------------------
// NT skinny: part[ks][m][j] = sum_{k in split ks} A[m][k] * B[j][k]
// A [M][K] bf16 (K % 64 == 0), B [RP][K] bf16.  A workgroup owns 64 rows and
// one K range; its 4 waves take interleaved K steps of 32 over that range
// (so together they stream contiguous memory), each computing 4 A fragments
// (16 rows) x RP/16 B fragments of v_mfma_f32_16x16x32_bf16 per step, and
// their four partial tiles are added in LDS in wave order.  Fragments come
// straight from global memory: A streams from HBM once, B is shared by all
// workgroups and stays in L2.
// ---------------------------------------------------------------------------
template <int RPT>
__global__ __launch_bounds__(256) void k_skinny_nt(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                   int64_t M, int K, int ksplit, int krange,
                                                   float* __restrict__ part) {
  constexpr int NJ = RPT / 16;
  __shared__ float red[64 * RPT];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t mblk = blockIdx.x / ksplit;
  const int ks = blockIdx.x - (int)(mblk * ksplit);
  const int64_t m0 = mblk * 64;
  const int k_lo = ks * krange;
  const int k_hi = min(K, k_lo + krange);
  const int li = lane & 15;
  const int kq = (lane >> 4) * 8;

  floatx4 acc[4][NJ];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[a][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* arow[4];
  bool aval[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t m = m0 + a * 16 + li;
    aval[a] = m < M;
    arow[a] = A + (aval[a] ? m : 0) * (int64_t)K;
  }
  for (int k = k_lo + 32 * wave; k < k_hi; k += 128) {
    bf16x8 af[4], bf[NJ];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (aval[a]) v = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)(arow[a] + k + kq)));
      af[a] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      bf[j] = __builtin_bit_cast(bf16x8, *(const uint4*)(B + (int64_t)(j * 16 + li) * K + k + kq));
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bf[j], acc[a][j], 0, 0, 0);
  }
  // D[i][jj]: lane holds column jj = lane%16, rows i = 4*(lane/16) + v.
  // Waves add their tiles into LDS one after another (fixed order).
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int idx = (a * 16 + 4 * (lane >> 4) + v) * RPT + j * 16 + li;
            red[idx] = (w == 0) ? acc[a][j][v] : red[idx] + acc[a][j][v];
          }
    }
    __syncthreads();
  }
  float* out = part + (int64_t)ks * M * RPT;
  for (int e = threadIdx.x; e < 64 * RPT; e += 256) {
    const int64_t m = m0 + e / RPT;
    if (m < M) out[m * RPT + (e % RPT)] = red[e];
  }
}

// out1[m][j] = bf16(alpha1 * sum_ks part) for j < r (row stride ld1), if out1;
// out2[m][j] = bf16(alpha2 * sum_ks part) for j < RP (row stride RP), if out2.
__global__ __launch_bounds__(256) void k_reduce_nt(const float* __restrict__ part, int64_t M, int RP, int r,
                                                   int ksplit, float alpha1, uint16_t* __restrict__ out1,
                                                   int ld1, float alpha2, uint16_t* __restrict__ out2) {
  const int64_t total = M * RP;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    float s = 0.f;
    for (int ks = 0; ks < ksplit; ++ks) s += part[(int64_t)ks * total + t];
    const int64_t m = t / RP;
    const int j = (int)(t - m * RP);
    if (out1 && j < r) out1[m * ld1 + j] = f32_to_bf16(alpha1 * s);
    if (out2) out2[t] = f32_to_bf16(alpha2 * s);
  }
}

// ---------------------------------------------------------------------------
// TN skinny: part[ms][j][n] = sum_{m in split ms} P[m][j] * Q[m][n]
// P [M][ldp] bf16 (columns >= r read as 0), Q [M][N] bf16.
// A workgroup owns 64 columns of n (16 per wave) and one token range.  Per
// chunk of TOK tokens it stages P^T [RP][TOK] in LDS (the A operand, shared by
// the 4 waves); each wave reads its Q fragments (B operand: 32 tokens x 16
// columns) with 2-byte loads, since the contraction runs along Q's rows.
// ---------------------------------------------------------------------------
template <int RPT>
__global__ __launch_bounds__(256) void k_skinny_tn(const uint16_t* __restrict__ P, int ldp, int r,
                                                   const uint16_t* __restrict__ Q, int64_t M, int N,
                                                   int msplit, int64_t mrange, float* __restrict__ part) {
  constexpr int NJ = RPT / 16;
  constexpr int TOK = (RPT <= 64) ? 128 : 32;
  __shared__ __attribute__((aligned(16))) uint16_t pt[RPT][TOK + 8];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nb = blockIdx.x / msplit;
  const int ms = blockIdx.x - nb * msplit;
  const int n = nb * 64 + wave * 16 + (lane & 15);
  const int64_t m_lo = (int64_t)ms * mrange;
  const int64_t m_hi = min(M, m_lo + mrange);
  const int li = lane & 15;
  const int kq = (lane >> 4) * 8;
  const bool nval = n < N;

  floatx4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int64_t m = m_lo; m < m_hi; m += TOK) {
    __syncthreads();
    for (int e = tid; e < RPT * TOK; e += 256) {
      const int mm = e / RPT;
      const int j = e - mm * RPT;
      const int64_t gm = m + mm;
      pt[j][mm] = (gm < m_hi && j < r) ? P[gm * ldp + j] : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < TOK / 32; ++c) {
      uint16_t q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t gm = m + c * 32 + kq + e;
        q[e] = (gm < m_hi && nval) ? Q[gm * N + n] : (uint16_t)0;
      }
      uint4 qv;
      qv.x = (uint32_t)q[0] | ((uint32_t)q[1] << 16);
      qv.y = (uint32_t)q[2] | ((uint32_t)q[3] << 16);
      qv.z = (uint32_t)q[4] | ((uint32_t)q[5] << 16);
      qv.w = (uint32_t)q[6] | ((uint32_t)q[7] << 16);
      const bf16x8 bq = __builtin_bit_cast(bf16x8, qv);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x8 af = *(const bf16x8*)&pt[j * 16 + li][c * 32 + kq];
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bq, acc[j], 0, 0, 0);
      }
    }
  }
  // D[i][col]: col = lane%16 -> n, rows i = 4*(lane/16) + v -> j
  float* out = part + (int64_t)ms * RPT * N;
  if (nval) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) out[(int64_t)(j * 16 + 4 * (lane >> 4) + v) * N + n] = acc[j][v];
  }
}

// out = alpha * sum_ms part[ms][j][n] for j < r, stored [r][N] (trans = 0)
// or [N][r] (trans = 1).
__global__ __launch_bounds__(256) void k_reduce_tn(const float* __restrict__ part, int RP, int r, int N,
                                                   int msplit, float alpha, int trans, float* __restrict__ out) {
  const int64_t total = (int64_t)r * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t j = t / N;
    const int64_t n = t - j * N;
    float s = 0.f;
    for (int ms = 0; ms < msplit; ++ms) s += part[((int64_t)ms * RP + j) * N + n];
    s *= alpha;
    if (trans) out[n * r + j] = s;
    else out[t] = s;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static unsigned grid_for(int64_t total, int64_t cap = 4096) {
  int64_t b = (total + 255) / 256;
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (unsigned)b;
}

hipError_t launch_pad_transpose(const uint16_t* in, int64_t si, int64_t sj, int64_t irows, int64_t jcols,
                                uint16_t* out, int64_t orows, int64_t ocols, hipStream_t st) {
  const int64_t total = orows * ocols;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pad_transpose, dim3(grid_for(total)), dim3(256), 0, st, in, si, sj, irows, jcols, out,
                     orows, ocols);
  return hipGetLastError();
}

// split-K factor for an NT skinny product over M rows (64 rows per workgroup):
// about 256 workgroups, each K range a multiple of 128 (4 waves x 32).
void plan_nt(int64_t M, int K, int* ksplit, int* krange) {
  const int64_t mblocks = (M + 63) / 64;
  int64_t ks = (256 + mblocks - 1) / (mblocks > 0 ? mblocks : 1);
  const int64_t kmax = (K + 127) / 128;
  if (ks > kmax) ks = kmax;
  if (ks < 1) ks = 1;
  int kr = (int)(((K + ks - 1) / ks + 127) / 128 * 128);
  ks = (K + kr - 1) / kr;
  *ksplit = (int)ks;
  *krange = kr;
}

// split-M factor for a TN skinny product with N output columns (64 per
// workgroup): about 256 workgroups, token ranges a multiple of 128.
void plan_tn(int64_t M, int N, int* msplit, int64_t* mrange) {
  const int64_t nblocks = (N + 63) / 64;
  int64_t ms = (256 + nblocks - 1) / nblocks;
  const int64_t mmax = (M + 127) / 128;
  if (ms > mmax) ms = mmax;
  if (ms < 1) ms = 1;
  int64_t mr = ((M + ms - 1) / ms + 127) / 128 * 128;
  if (mr < 128) mr = 128;
  ms = (M + mr - 1) / mr;
  if (ms < 1) ms = 1;
  *msplit = (int)ms;
  *mrange = mr;
}

#define NF4K_RP_SWITCH(RP, LAUNCH) \
  switch (RP) {                    \
    case 16: LAUNCH(16); break;    \
    case 32: LAUNCH(32); break;    \
    case 48: LAUNCH(48); break;    \
    case 64: LAUNCH(64); break;    \
    case 80: LAUNCH(80); break;    \
    case 96: LAUNCH(96); break;    \
    case 112: LAUNCH(112); break;  \
    case 128: LAUNCH(128); break;  \
    case 144: LAUNCH(144); break;  \
    case 160: LAUNCH(160); break;  \
    case 176: LAUNCH(176); break;  \
    case 192: LAUNCH(192); break;  \
    case 208: LAUNCH(208); break;  \
    case 224: LAUNCH(224); break;  \
    case 240: LAUNCH(240); break;  \
    case 256: LAUNCH(256); break;  \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_skinny_nt(const uint16_t* A, const uint16_t* B, int64_t M, int K, int RP, float* part,
                            int ksplit, int krange, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int64_t mblocks = (M + 63) / 64;
  const dim3 gr((unsigned)(mblocks * ksplit)), bl(256);
#define L_NT(R) hipLaunchKernelGGL(k_skinny_nt<R>, gr, bl, 0, st, A, B, M, K, ksplit, krange, part)
  NF4K_RP_SWITCH(RP, L_NT)
#undef L_NT
  return hipGetLastError();
}

hipError_t launch_reduce_nt(const float* part, int64_t M, int RP, int r, int ksplit, float alpha1, uint16_t* out1,
                            int ld1, float alpha2, uint16_t* out2, hipStream_t st) {
  const int64_t total = M * RP;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_reduce_nt, dim3(grid_for(total)), dim3(256), 0, st, part, M, RP, r, ksplit, alpha1, out1,
                     ld1, alpha2, out2);
  return hipGetLastError();
}

hipError_t launch_skinny_tn(const uint16_t* P, int ldp, int r, const uint16_t* Q, int64_t M, int N, int RP,
                            float* part, int msplit, int64_t mrange, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int nblocks = (N + 63) / 64;
  const dim3 gr((unsigned)(nblocks * msplit)), bl(256);
#define L_TN(R) hipLaunchKernelGGL(k_skinny_tn<R>, gr, bl, 0, st, P, ldp, r, Q, M, N, msplit, mrange, part)
  NF4K_RP_SWITCH(RP, L_TN)
#undef L_TN
  return hipGetLastError();
}

hipError_t launch_reduce_tn(const float* part, int RP, int r, int N, int msplit, float alpha, int trans, float* out,
                            hipStream_t st) {
  const int64_t total = (int64_t)r * N;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_reduce_tn, dim3(grid_for(total)), dim3(256), 0, st, part, RP, r, N, msplit, alpha, trans,
                     out);
  return hipGetLastError();
}

}  // namespace nf4k
