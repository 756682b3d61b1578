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
// long contraction is split over workgroups so that enough loads are in
// flight to cover HBM latency.  Each split writes an fp32 partial; the last
// workgroup of a tile to finish (found with an agent-scope counter) adds the
// partials in split order and writes the result, so results do not depend
// on scheduling and no second launch is needed.  Counters start at zero
// (k_prep clears them) and are reset by the workgroup that used them.
//
// Internally r is padded to RP = 16*ceil(r/16); padded rows/columns are zero.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace nf4k {

// ---------------------------------------------------------------------------
// k_prep: the layout copies of the adapters and the clearing of counters or
// outputs, all in one launch.  blockIdx.y selects the job.
//   pad job:  out[i][j] = (i < irows && j < jcols) ? in[i*si + j*sj] : 0
//   zero job: p[0 .. n) = 0 (32-bit words)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_prep(PrepArgs a) {
  const int job = blockIdx.y;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (job < kPrepPads) {
    const PadJob& p = a.pad[job];
    const int64_t total = p.orows * p.ocols;
    for (int64_t t = t0; t < total; t += stride) {
      const int64_t i = t / p.ocols;
      const int64_t j = t - i * p.ocols;
      p.out[t] = (i < p.irows && j < p.jcols) ? p.in[i * p.si + j * p.sj] : (uint16_t)0;
    }
  } else {
    const ZeroJob& z = a.zero[job - kPrepPads];
    for (int64_t t = t0; t < z.n; t += stride) z.p[t] = 0u;
  }
}

// Split partials are exchanged between workgroups through agent-scope
// atomic stores and loads: these bypass the non-coherent L2 lines, so a value
// written on one XCD is read back correctly on another without a device-wide
// fence (which on this chip writes back and invalidates a whole L2).
__device__ __forceinline__ void st_shared_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_shared_partial(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// sum_{q < n} part[q * slab + off], added in q order; the loads are issued
// eight at a time so the sum costs a few memory round trips, not n.
__device__ __forceinline__ float sum_partials(const float* part, int64_t slab, int64_t off, int n) {
  float sum = 0.f;
  for (int q0 = 0; q0 < n; q0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (q0 + u < n) ? ld_shared_partial(part + (int64_t)(q0 + u) * slab + off) : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  return sum;
}

// Split-reduction handshake: every thread's partial stores have completed
// (vmcnt 0) before the barrier, so they are complete before thread 0 counts
// this workgroup.  Returns true in the last workgroup of a tile, which then
// reads every split's partial with ld_shared_partial.
__device__ __forceinline__ bool last_arrival(unsigned* cnt, int nsplit) {
  __shared__ int s_last;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(nsplit - 1);
  __syncthreads();
  if (!s_last) return false;
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// ---------------------------------------------------------------------------
// NT skinny: out[m][j] = alpha * sum_k A[m][k] * B[j][k]
// A [M][K] bf16 (K % 64 == 0), B [RP][K] bf16.  A workgroup owns 64 rows and
// one K range; its 4 waves take interleaved K steps of 32 over that range
// (together they stream contiguous memory), U steps at a time with all loads
// issued before the MFMAs, each step 4 A fragments (16 rows) x RP/16 B
// fragments of v_mfma_f32_16x16x32_bf16.  The four wave tiles are added in
// LDS in wave order.  A streams from HBM once; B is shared by every
// workgroup and stays in L2.
// Outputs: out1[m][j] = bf16(alpha1 * sum) for j < r (row stride ld1), if
// out1; out2[m][j] = bf16(alpha2 * sum) for j < RP (row stride RP), if out2.
// ---------------------------------------------------------------------------
template <int RPT>
__global__ __launch_bounds__(256) void k_skinny_nt(NtArgs p) {
  constexpr int NJ = RPT / 16;
  constexpr int U = RPT <= 32 ? 4 : (RPT <= 64 ? 2 : 1);
  __shared__ float red[64 * RPT];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t mblk = blockIdx.x / p.ksplit;
  const int ks = blockIdx.x - (int)(mblk * p.ksplit);
  const int64_t m0 = mblk * 64;
  const int64_t M = p.M;
  const int K = p.K;
  const int k_lo = ks * p.krange;
  const int k_hi = min(K, k_lo + p.krange);
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
    arow[a] = p.A + (aval[a] ? m : 0) * (int64_t)K;
  }
  for (int k0 = k_lo + 32 * wave; k0 < k_hi; k0 += 128 * U) {
    bf16x8 af[U][4], bf[U][NJ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 128 * u;
      const bool kv = k < k_hi;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (kv && aval[a]) v = __builtin_nontemporal_load((const u32x4*)(arow[a] + k + kq));
        af[u][a] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (kv) v = *(const u32x4*)(p.B + (int64_t)(j * 16 + li) * K + k + kq);
        bf[u][j] = __builtin_bit_cast(bf16x8, v);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][a], bf[u][j], acc[a][j], 0, 0, 0);
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
  auto emit = [&](int e, float sum) {
    const int64_t m = m0 + e / RPT;
    const int j = e % RPT;
    if (p.out1 && j < p.r) p.out1[m * p.ld1 + j] = f32_to_bf16(p.alpha1 * sum);
    if (p.out2) p.out2[m * RPT + j] = f32_to_bf16(p.alpha2 * sum);
  };
  if (p.ksplit == 1) {
    for (int e = threadIdx.x; e < 64 * RPT; e += 256)
      if (m0 + e / RPT < M) emit(e, red[e]);
    return;
  }
  const int64_t slab = M * RPT;
  float* mine = p.part + (int64_t)ks * slab;
  for (int e = threadIdx.x; e < 64 * RPT; e += 256) {
    const int64_t m = m0 + e / RPT;
    if (m < M) st_shared_partial(mine + m * RPT + (e % RPT), red[e]);
  }
  if (!last_arrival(p.cnt + mblk, p.ksplit)) return;
  for (int e = threadIdx.x; e < 64 * RPT; e += 256) {
    const int64_t m = m0 + e / RPT;
    if (m >= M) continue;
    const int64_t off = m * RPT + (e % RPT);
    emit(e, sum_partials(p.part, slab, off, p.ksplit));
  }
}

// ---------------------------------------------------------------------------
// TN skinny: out[j][n] = alpha * sum_m P[m][j] * Q[m][n]   (j < r)
// P [M][ldp] bf16 with ldp % 8 == 0 and columns r .. ceil8(r)-1 zero (P is
// read in 16-byte chunks of 8 columns; chunks at or past r are not read),
// Q [M][N] bf16 (N % 64 == 0).
// The contraction runs along the rows of both operands, so a workgroup (64
// columns of Q, one token range) loads chunks of TOK tokens of Q and P with
// coalesced 16-byte loads, the next chunk in registers while the current one
// is multiplied, and writes them transposed into LDS ([column][token], rows
// padded by 8 elements so the 16-byte fragment reads hit distinct banks).
// Wave w then takes columns 16w..16w+15: B fragment = 32 tokens of one Q
// column, A fragments = 32 tokens of 16 P columns, v_mfma_f32_16x16x32_bf16.
// Stored [r][N] (trans = 0) or [N][r] (trans = 1), fp32.
// ---------------------------------------------------------------------------
template <int RPT>
struct TnShape {
  static constexpr int TOK = RPT <= 64 ? 256 : (RPT <= 128 ? 128 : 64);  // tokens per chunk
  static constexpr int LDT = TOK + 8;                                     // LDS row length (elements)
  static constexpr int QCH = TOK * 64 / 8 / 256;                          // 16-byte Q chunks per thread
  static constexpr int PCH = (TOK * RPT / 8 + 255) / 256;                 // 16-byte P chunks per thread (ceil)
};

template <int RPT>
__global__ __launch_bounds__(256) void k_skinny_tn(TnArgs p) {
  using S = TnShape<RPT>;
  constexpr int NJ = RPT / 16;
  constexpr int TOK = S::TOK, LDT = S::LDT, QCH = S::QCH, PCH = S::PCH;
  static_assert(QCH * 256 * 8 == TOK * 64, "chunk split");
  constexpr int PCHUNKS = TOK * RPT / 8;
  __shared__ __attribute__((aligned(16))) uint16_t qt[64 * LDT];
  __shared__ __attribute__((aligned(16))) uint16_t pt[RPT * LDT];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nb = blockIdx.x / p.msplit;
  const int ms = blockIdx.x - nb * p.msplit;
  const int n0 = nb * 64;
  const int64_t m_lo = (int64_t)ms * p.mrange;
  const int64_t m_hi = min(p.M, m_lo + p.mrange);
  const int N = p.N;

  u32x4 qreg[QCH], preg[PCH];
  auto load_chunk = [&](int64_t m) {
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int row = (tid >> 3) + 32 * i;
      const int col = n0 + (tid & 7) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (m + row < m_hi && col < N) v = __builtin_nontemporal_load((const u32x4*)(p.Q + (m + row) * N + col));
      qreg[i] = v;
    }
#pragma unroll
    for (int i = 0; i < PCH; ++i) {
      const int e = tid + 256 * i;
      const int row = e / (RPT / 8);
      const int j0 = (e % (RPT / 8)) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (e < PCHUNKS && m + row < m_hi && j0 < p.r) v = *(const u32x4*)(p.P + (m + row) * p.ldp + j0);
      preg[i] = v;
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int row = (tid >> 3) + 32 * i;
      const int c0 = (tid & 7) * 8;
#pragma unroll
      for (int t = 0; t < 8; ++t) qt[(c0 + t) * LDT + row] = (uint16_t)(qreg[i][t >> 1] >> (16 * (t & 1)));
    }
#pragma unroll
    for (int i = 0; i < PCH; ++i) {
      const int e = tid + 256 * i;
      const int row = e / (RPT / 8);
      const int j0 = (e % (RPT / 8)) * 8;
      if (e < PCHUNKS) {
#pragma unroll
        for (int t = 0; t < 8; ++t) pt[(j0 + t) * LDT + row] = (uint16_t)(preg[i][t >> 1] >> (16 * (t & 1)));
      }
    }
  };

  floatx4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int li = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int ncol = wave * 16 + li;

  if (m_lo < m_hi) load_chunk(m_lo);
  for (int64_t m = m_lo; m < m_hi; m += TOK) {
    __syncthreads();  // previous chunk's fragment reads are done
    store_chunk();
    if (m + TOK < m_hi) load_chunk(m + TOK);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < TOK / 32; ++c) {
      const bf16x8 bq = *(const bf16x8*)&qt[ncol * LDT + c * 32 + kq];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x8 af = *(const bf16x8*)&pt[(j * 16 + li) * LDT + c * 32 + kq];
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bq, acc[j], 0, 0, 0);
      }
    }
  }
  // D[i][col]: col = lane%16 -> n, rows i = 4*(lane/16) + v -> j
  const int n = n0 + ncol;
  auto emit = [&](int j, int nn, float sum) {
    if (j >= p.r || nn >= N) return;
    if (p.trans) p.out[(int64_t)nn * p.r + j] = p.alpha * sum;
    else p.out[(int64_t)j * N + nn] = p.alpha * sum;
  };
  if (p.msplit == 1) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) emit(j * 16 + 4 * (lane >> 4) + v, n, acc[j][v]);
    return;
  }
  const int64_t slab = (int64_t)RPT * N;
  float* mine = p.part + (int64_t)ms * slab;
  if (n < N) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) st_shared_partial(mine + (int64_t)(j * 16 + 4 * (lane >> 4) + v) * N + n, acc[j][v]);
  }
  if (!last_arrival(p.cnt + nb, p.msplit)) return;
  for (int e = tid; e < RPT * 64; e += 256) {
    const int j = e >> 6;
    const int nn = n0 + (e & 63);
    if (j >= p.r || nn >= N) continue;
    const int64_t off = (int64_t)j * N + nn;
    emit(j, nn, sum_partials(p.part, slab, off, p.msplit));
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_prep(const PrepArgs& a, hipStream_t st) {
  int64_t most = 0;
  for (int i = 0; i < kPrepPads; ++i) most = std::max(most, a.pad[i].orows * a.pad[i].ocols);
  for (int i = 0; i < kPrepZeros; ++i) most = std::max(most, a.zero[i].n);
  if (most == 0) return hipSuccess;
  int64_t bx = (most + 255) / 256;
  if (bx > 1024) bx = 1024;
  hipLaunchKernelGGL(k_prep, dim3((unsigned)bx, kPrepPads + kPrepZeros), dim3(256), 0, st, a);
  return hipGetLastError();
}

// split-K factor for an NT skinny product over M rows (64 rows per
// workgroup): about 512 workgroups, each K range a multiple of 128.
void plan_nt(int64_t M, int K, int* ksplit, int* krange) {
  const int64_t mblocks = (M + 63) / 64;
  int64_t ks = (512 + mblocks - 1) / (mblocks > 0 ? mblocks : 1);
  const int64_t kmax = (K + 127) / 128;
  if (ks > kmax) ks = kmax;
  if (ks < 1) ks = 1;
  int kr = (int)(((K + ks - 1) / ks + 127) / 128 * 128);
  ks = (K + kr - 1) / kr;
  *ksplit = (int)ks;
  *krange = kr;
}

// split-M factor for a TN skinny product with N output columns (64 per
// workgroup): about 512 workgroups, token ranges a multiple of 256 (a whole
// number of chunks for every rank).
void plan_tn(int64_t M, int N, int* msplit, int64_t* mrange) {
  const int64_t nblocks = (N + 63) / 64;
  int64_t ms = (512 + nblocks - 1) / nblocks;
  const int64_t mmax = (M + 255) / 256;
  if (ms > mmax) ms = mmax;
  if (ms < 1) ms = 1;
  int64_t mr = ((M + ms - 1) / ms + 255) / 256 * 256;
  if (mr < 256) mr = 256;
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

hipError_t launch_skinny_nt(const NtArgs& a, int RP, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const int64_t mblocks = (a.M + 63) / 64;
  const dim3 gr((unsigned)(mblocks * a.ksplit)), bl(256);
#define L_NT(R) hipLaunchKernelGGL(k_skinny_nt<R>, gr, bl, 0, st, a)
  NF4K_RP_SWITCH(RP, L_NT)
#undef L_NT
  return hipGetLastError();
}

hipError_t launch_skinny_tn(const TnArgs& a, int RP, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const int nblocks = (a.N + 63) / 64;
  const dim3 gr((unsigned)(nblocks * a.msplit)), bl(256);
#define L_TN(R) hipLaunchKernelGGL(k_skinny_tn<R>, gr, bl, 0, st, a)
  NF4K_RP_SWITCH(RP, L_TN)
#undef L_TN
  return hipGetLastError();
}

}  // namespace nf4k
