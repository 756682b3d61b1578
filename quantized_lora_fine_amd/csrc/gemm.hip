// Fused NF4-dequant bf16 MFMA GEMM for the QLoRA linear (gfx950).
//
//   C[M][N] = A[M][K] * B[N][K]^T  +  A2[M][R] * B2[N][R]^T      (fp32 accumulate)
//
// Forward  (MODE_FWD): A = X [M][h], B = w_hat(W_st) with W_st [o][h]
//                      (N = o, K = h), tail A2 = s*T [M][R], B2 = L2^T [o][R].
// Input grad (MODE_DX): A = dY [M][o], B = w_hat(W_st)^T (N = h, K = o),
//                      tail A2 = G [M][R], B2 = L1 [h][R].
//
// This is equation (3) of "QLoRA: How to fine-tune large language models
// with less memory" with the base dequantized to bf16 right before the
// product ("1. NormalFloat": weights are reconstructed into bf16 for the
// matmul) and the rank-R adapter product folded in as extra K columns of the
// same output tile, so the adapter term costs no extra pass over C.  The
// dequantized W tile exists only in LDS: packed 4-bit codes and scales are
// the only weight bytes read from HBM.
//
// Tiling: 256 x 128 output tile per 256-thread workgroup (4 wave64s, 2 x 2,
// each wave 128 x 64 as 4 x 2 v_mfma_f32_32x32x16_bf16), K step 64 (one NF4
// block per W row per step), double-buffered LDS (96 KiB): the global loads
// of step k+1 are issued before the MFMAs of step k and written to the other
// buffer after them, one barrier per step.  LDS rows are 128 B (64 bf16) in
// 8 chunks of 16 B with an XOR swizzle so that the 16-byte fragment reads
// are bank-conflict free.  Workgroup ids are remapped so the tiles that run
// together on one XCD share the same rows of A (its L2 keeps that panel).
#include "common.hpp"
#include "launch.hpp"

namespace nf4k {

constexpr int GBM = 256;
constexpr int GBN = 128;
constexpr int GBK = 64;
constexpr int GNT = 256;



struct GemmArgs {
  const uint16_t* A;
  const uint8_t* codes;
  const void* absmax;
  const float* dqs;
  const uint16_t* A2;
  const uint16_t* B2;
  uint16_t* C;
  int64_t M;
  int N;
  int K;
  int R;  // tail width, a multiple of 16 (0 = no tail)
  int tiles_n;
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

template <int MODE, bool DQ>
__global__ __launch_bounds__(GNT) void k_nf4_gemm(GemmArgs p, NF4Consts cst) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (GBM + GBN) * 128];
  __shared__ float tab[16];
  uint8_t* const As = smem;
  uint8_t* const Bs = smem + 2 * GBM * 128;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;

  int lid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) lid = (lid & 7) * (nwg >> 3) + (lid >> 3);
  const int tm = lid / p.tiles_n;
  const int tn = lid - tm * p.tiles_n;
  const int64_t m0 = (int64_t)tm * GBM;
  const int n0 = tn * GBN;
  const int64_t M = p.M;
  const int N = p.N;
  const int K = p.K;

  if (tid < 16) tab[tid] = cst.table[tid];

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // ---- A tile: 256 rows x 64 bf16; thread loads 8 chunks of 16 B ----
  const int a_kc = tid & 7;
  const int a_r0 = tid >> 3;  // rows a_r0 + 32*i
  uint4 areg[8];
  auto load_A = [&](const uint16_t* src, int ld, int col0, int width) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t gm = m0 + a_r0 + 32 * i;
      const int col = col0 + a_kc * 8;
      if (gm < M && a_kc * 8 < width) {
        areg[i] = *(const uint4*)(src + gm * ld + col);
      } else {
        areg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_A = [&](int buf) {
    uint8_t* dst = As + buf * GBM * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4*)(dst + lds_off(a_r0 + 32 * i, a_kc)) = areg[i];
  };

  // ---- B tile producer ----
  // FWD: thread (n = tid>>1, half = tid&1) dequantizes 32 consecutive k of W row n0+n.
  // DX : thread (og = tid>>4, hc = tid&15) dequantizes 4 W rows (k) x 8 columns (n).
  uint4 creg4;
  uint32_t creg[4];
  float sreg[4];
  auto load_scale = [&](int64_t blk) -> float {
    if constexpr (DQ) {
      return (float)((const uint8_t*)p.absmax)[blk] * p.dqs[blk >> 8];
    } else {
      return ((const float*)p.absmax)[blk];
    }
  };
  auto load_B = [&](int kt) {
    if constexpr (MODE == MODE_FWD) {
      const int n = tid >> 1;
      const int half = tid & 1;
      const int gn = n0 + n;
      if (gn < N) {
        creg4 = *(const uint4*)(p.codes + (int64_t)gn * (K >> 1) + kt * 32 + half * 16);
        sreg[0] = load_scale((int64_t)gn * (K >> 6) + kt);
      } else {
        creg4 = make_uint4(0, 0, 0, 0);
        sreg[0] = 0.f;
      }
    } else {
      const int og = tid >> 4;
      const int hc = tid & 15;
      const int gh = n0 + hc * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t ko = (int64_t)kt * GBK + og * 4 + i;
        if (gh < N) {
          creg[i] = *(const uint32_t*)(p.codes + ko * (N >> 1) + (gh >> 1));
          sreg[i] = load_scale(ko * (N >> 6) + (gh >> 6));
        } else {
          creg[i] = 0;
          sreg[i] = 0.f;
        }
      }
    }
  };
  auto store_B = [&](int buf) {
    uint8_t* dst = Bs + buf * GBN * 128;
    if constexpr (MODE == MODE_FWD) {
      const int n = tid >> 1;
      const int half = tid & 1;
      const uint32_t wds[4] = {creg4.x, creg4.y, creg4.z, creg4.w};
      const float sc = sreg[0];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = wds[j];
        uint4 o;
        o.x = pack_bf16x2(tab[w & 15u] * sc, tab[(w >> 4) & 15u] * sc);
        o.y = pack_bf16x2(tab[(w >> 8) & 15u] * sc, tab[(w >> 12) & 15u] * sc);
        o.z = pack_bf16x2(tab[(w >> 16) & 15u] * sc, tab[(w >> 20) & 15u] * sc);
        o.w = pack_bf16x2(tab[(w >> 24) & 15u] * sc, tab[w >> 28] * sc);
        *(uint4*)(dst + lds_off(n, half * 4 + j)) = o;
      }
    } else {
      const int og = tid >> 4;
      const int hc = tid & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v0 = tab[(creg[0] >> (4 * e)) & 15u] * sreg[0];
        const float v1 = tab[(creg[1] >> (4 * e)) & 15u] * sreg[1];
        const float v2 = tab[(creg[2] >> (4 * e)) & 15u] * sreg[2];
        const float v3 = tab[(creg[3] >> (4 * e)) & 15u] * sreg[3];
        const int row = hc * 8 + e;
        uint2 o;
        o.x = pack_bf16x2(v0, v1);
        o.y = pack_bf16x2(v2, v3);
        *(uint2*)(dst + row * 128 + (((og >> 1) ^ swz(row)) << 4) + (og & 1) * 8) = o;
      }
    }
  };

  // ---- MFMA on one LDS buffer: nk16 steps of K = 16 ----
  auto compute = [&](int buf, int nk16) {
    const uint8_t* Ab = As + buf * GBM * 128;
    const uint8_t* Bb = Bs + buf * GBN * 128;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < nk16) {
        const int chunk = kk * 2 + (lane >> 5);
        bf16x8 af[4], bf[2];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          af[mi] = *(const bf16x8*)(Ab + lds_off(wm * 128 + mi * 32 + (lane & 31), chunk));
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          bf[ni] = *(const bf16x8*)(Bb + lds_off(wn * 64 + ni * 32 + (lane & 31), chunk));
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[ni], af[mi], acc[mi][ni], 0, 0, 0);
      }
    }
  };

  const int KT = K / GBK;
  __syncthreads();  // tab[]
  if (KT > 0) {
    load_A(p.A, K, 0, GBK);
    load_B(0);
    store_A(0);
    store_B(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < KT;
      if (more) {
        load_A(p.A, K, (kt + 1) * GBK, GBK);
        load_B(kt + 1);
      }
      compute(cur, 4);
      if (more) {
        store_A(cur ^ 1);
        store_B(cur ^ 1);
      }
      __syncthreads();
    }
  }

  // ---- adapter tail: R extra K columns from A2 [M][R] and B2 [N][R] ----
  for (int c0 = 0; c0 < p.R; c0 += GBK) {
    const int width = min(GBK, p.R - c0);
    load_A(p.A2, p.R, c0, width);
    store_A(0);
    {
      // B2 rows n0..n0+127: thread loads 4 chunks (row = tid>>1, chunks (tid&1)*4 + j)
      const int n = tid >> 1;
      const int half = tid & 1;
      const int gn = n0 + n;
      uint8_t* dst = Bs;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kc = half * 4 + j;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (gn < N && kc * 8 < width) v = *(const uint4*)(p.B2 + (int64_t)gn * p.R + c0 + kc * 8);
        *(uint4*)(dst + lds_off(n, kc)) = v;
      }
    }
    __syncthreads();
    compute(0, width >> 4);
    __syncthreads();
  }

  // ---- epilogue: D[n][m] per MFMA; lane holds m = l%32 and n = 8*(v/4) + 4*(l/32) + v%4 ----
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int64_t m = m0 + wm * 128 + mi * 32 + (lane & 31);
    if (m < M) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * 64 + ni * 32 + 8 * g + 4 * (lane >> 5);
          if (n < N) {
            uint2 o;
            o.x = pack_bf16x2(acc[mi][ni][4 * g + 0], acc[mi][ni][4 * g + 1]);
            o.y = pack_bf16x2(acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]);
            *(uint2*)(p.C + m * N + n) = o;
          }
        }
      }
    }
  }
}

hipError_t launch_nf4_gemm(int mode, bool dq, const uint16_t* A, const uint8_t* codes, const void* absmax,
                           const float* dqs, const uint16_t* A2, const uint16_t* B2, int R, uint16_t* C,
                           int64_t M, int N, int K, const NF4Consts& c, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmArgs p;
  p.A = A;
  p.codes = codes;
  p.absmax = absmax;
  p.dqs = dqs;
  p.A2 = A2;
  p.B2 = B2;
  p.C = C;
  p.M = M;
  p.N = N;
  p.K = K;
  p.R = R;
  const int64_t tiles_m = (M + GBM - 1) / GBM;
  p.tiles_n = (N + GBN - 1) / GBN;
  const int64_t nwg = tiles_m * p.tiles_n;
  const dim3 gr((unsigned)nwg), bl(GNT);
  if (mode == MODE_FWD) {
    if (dq) hipLaunchKernelGGL((k_nf4_gemm<MODE_FWD, true>), gr, bl, 0, st, p, c);
    else hipLaunchKernelGGL((k_nf4_gemm<MODE_FWD, false>), gr, bl, 0, st, p, c);
  } else {
    if (dq) hipLaunchKernelGGL((k_nf4_gemm<MODE_DX, true>), gr, bl, 0, st, p, c);
    else hipLaunchKernelGGL((k_nf4_gemm<MODE_DX, false>), gr, bl, 0, st, p, c);
  }
  return hipGetLastError();
}

}  // namespace nf4k
