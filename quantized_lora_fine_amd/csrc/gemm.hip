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
// block per W row per step), double-buffered LDS.
//   * A (X or dY) goes straight from global memory into LDS with
//     buffer_load_dwordx4 ... lds, one K step ahead; rows past M read as zero
//     through the buffer descriptor's range check, so the loop has no branches.
//   * W codes and scales are loaded into registers two K steps ahead; while
//     the MFMAs of step k run, the codes of step k+1 are dequantized into the
//     other B buffer a quarter at a time between the K=16 MFMA groups, so the
//     dequant VALU work hides under the matrix cores.
//   * dequant: each code byte (two NF4 codes) indexes a 256-entry LDS table of
//     fp32 value pairs; the pair is multiplied by the block scale and packed to
//     bf16 with v_cvt_pk_bf16_f32 (round to nearest even), exactly the bf16 of
//     the fp32 dequantized weight.
//   * LDS rows are 128 B (64 bf16) in 8 chunks of 16 B with an XOR swizzle so
//     that the 16-byte MFMA fragment reads are bank-conflict free.
//   * Workgroup ids are remapped so the tiles that run together on one XCD
//     share the same rows of A (its L2 keeps that panel).
#include "common.hpp"
#include "launch.hpp"

namespace nf4k {

constexpr int GBM = 256;
constexpr int GBN = 128;
constexpr int GBK = 64;
constexpr int GNT = 256;
constexpr uint32_t kRsrcFlags = 0x00020000u;  // raw buffer, gfx9-family dword3
constexpr uint32_t kOOB = 0x80000000u;        // an offset past every buffer's range

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
  int64_t nblocks;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcFlags);
}

template <int MODE, bool DQ>
__global__ __launch_bounds__(GNT) void k_nf4_gemm(GemmArgs p, NF4Consts cst) {
  // separate arrays per buffer: the compiler then knows a direct-to-LDS load
  // into one A buffer cannot alias fragment reads from the other, and does not
  // wait for the next tile's loads before reading the current one
  __shared__ __attribute__((aligned(16))) uint8_t As0[GBM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t As1[GBM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Bs0[GBN * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Bs1[GBN * 128];
  __shared__ __attribute__((aligned(16))) float2 ptab[256];

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
  const int KT = K / GBK;

  // byte -> (table[low nibble], table[high nibble]): element 2t sits in the low nibble
  ptab[tid] = make_float2(cst.table[tid & 15], cst.table[tid >> 4]);

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // ---- A: direct global -> LDS, 8 x 1 KiB per wave per K step ----
  const int64_t arows = (M - m0) < GBM ? (M - m0) : GBM;
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.A + m0 * K, (uint32_t)(arows * K * 2));
  // lane l of the wave's i-th instruction fills LDS row r = (wave*8+i)*8 + l/8,
  // physical chunk l%8, i.e. logical chunk (l%8) ^ swz(r)
  uint32_t a_voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (wave * 8 + i) * 8 + (lane >> 3);
    a_voff[i] = (uint32_t)(r * K * 2 + (((lane & 7) ^ swz(r)) << 4));
  }
  auto issue_A = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint8_t* dst = (buf ? As1 : As0) + (wave * 8 + i) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)dst, 16, a_voff[i] + kt * 128, 0, 0, 0);
    }
  };

  // ---- W codes + scales into registers (two register sets, two steps ahead) ----
  __amdgpu_buffer_rsrc_t c_rsrc, s_rsrc, q_rsrc;
  uint32_t c_voff[4], s_voff[4];
  if constexpr (MODE == MODE_FWD) {
    // thread (n = tid>>1, half = tid&1): 32 consecutive codes of W row n0+n
    const int n = tid >> 1;
    const int nrows = (N - n0) < GBN ? (N - n0) : GBN;
    c_rsrc = make_rsrc(p.codes + (int64_t)n0 * (K >> 1), (uint32_t)((int64_t)nrows * (K >> 1)));
    c_voff[0] = (uint32_t)(n * (K >> 1) + (tid & 1) * 16);
    s_voff[0] = (uint32_t)(n0 + n) * (uint32_t)(K >> 6);  // block index at kt = 0
  } else {
    // thread (og = tid>>4, hc = tid&15): rows kt*64 + og*4 + i (i < 4), columns n0 + hc*8 .. +8
    const int og = tid >> 4;
    const int hc = tid & 15;
    const bool ok = n0 + hc * 8 < N;
    c_rsrc = make_rsrc(p.codes, (uint32_t)(p.nblocks * 32));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c_voff[i] = ok ? (uint32_t)((og * 4 + i) * (N >> 1) + ((n0 + hc * 8) >> 1)) : kOOB;
      s_voff[i] = ok ? (uint32_t)((og * 4 + i) * (N >> 6) + ((n0 + hc * 8) >> 6)) : kOOB;
    }
  }
  s_rsrc = make_rsrc(p.absmax, (uint32_t)(p.nblocks * (DQ ? 1 : 4)));
  q_rsrc = make_rsrc(p.dqs, (uint32_t)(DQ ? ((p.nblocks + 255) / 256) * 4 : 0));

  u32x4 creg[2];
  uint32_t sraw[2][4];   // fp32 absmax bits, or the 8-bit scale code
  float sstep[2][4];     // double quant: the group's fp32 step
  // The scale is formed where it is used (in the dequant), not here, so that
  // nothing waits on these loads before the step that consumes them.
  auto load_scale = [&](uint32_t blk, int set, int i) {
    if constexpr (DQ) {
      sraw[set][i] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, blk, 0, 0);
      sstep[set][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(q_rsrc, (blk >> 8) * 4, 0, 0));
    } else {
      sraw[set][i] = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, blk * 4, 0, 0);
    }
  };
  auto scale = [&](int set, int i) -> float {
    if constexpr (DQ) {
      return (float)sraw[set][i] * sstep[set][i];
    } else {
      return __builtin_bit_cast(float, sraw[set][i]);
    }
  };
  // Out-of-range rows/columns carry offsets >= 2^31, past every descriptor's
  // range (all buffers are < 2 GiB), so their codes and scales read as 0.
  auto issue_W = [&](int kt, int set) {
    if constexpr (MODE == MODE_FWD) {
      creg[set] = __builtin_amdgcn_raw_buffer_load_b128(c_rsrc, c_voff[0] + kt * 32, 0, 0);
      load_scale(s_voff[0] + kt, set, 0);
    } else {
      const uint32_t drow = (uint32_t)kt * 64u * (uint32_t)(N >> 1);
      const uint32_t dblk = (uint32_t)kt * 64u * (uint32_t)(N >> 6);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        creg[set][i] = __builtin_amdgcn_raw_buffer_load_b32(c_rsrc, c_voff[i] + drow, 0, 0);
        load_scale(s_voff[i] + dblk, set, i);
      }
    }
  };
  // vector-memory instructions issue_W emits (what may stay in flight at a step's end)
  constexpr int kWLoads = (MODE == MODE_FWD) ? (DQ ? 3 : 2) : (DQ ? 12 : 8);
  constexpr int kWaitW = (kWLoads & 15) | ((kWLoads >> 4) << 14) | (0x7 << 4) | (0xF << 8);

  // dequantize quarter q (0..3) of the B tile held in register set `set` into LDS buffer `buf`
  auto dequant_quarter = [&](int set, int buf, int q) {
    uint8_t* dst = buf ? Bs1 : Bs0;
    if constexpr (MODE == MODE_FWD) {
      const uint32_t w = creg[set][q];
      const float sc = scale(set, 0);
      const float2 t0 = ptab[w & 0xFFu], t1 = ptab[(w >> 8) & 0xFFu], t2 = ptab[(w >> 16) & 0xFFu],
                   t3 = ptab[w >> 24];
      uint4 o;
      o.x = pack_bf16x2(t0.x * sc, t0.y * sc);
      o.y = pack_bf16x2(t1.x * sc, t1.y * sc);
      o.z = pack_bf16x2(t2.x * sc, t2.y * sc);
      o.w = pack_bf16x2(t3.x * sc, t3.y * sc);
      *(uint4*)(dst + lds_off(tid >> 1, (tid & 1) * 4 + q)) = o;
    } else {
      // byte q of each of the 4 row words: columns hc*8 + 2q and +1
      const int og = tid >> 4;
      const int hc = tid & 15;
      float2 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 t = ptab[(creg[set][i] >> (8 * q)) & 0xFFu];
        const float sc = scale(set, i);
        v[i] = make_float2(t.x * sc, t.y * sc);
      }
      const int row0 = hc * 8 + 2 * q;
      uint2 e0, e1;
      e0.x = pack_bf16x2(v[0].x, v[1].x);
      e0.y = pack_bf16x2(v[2].x, v[3].x);
      e1.x = pack_bf16x2(v[0].y, v[1].y);
      e1.y = pack_bf16x2(v[2].y, v[3].y);
      *(uint2*)(dst + row0 * 128 + (((og >> 1) ^ swz(row0)) << 4) + (og & 1) * 8) = e0;
      *(uint2*)(dst + (row0 + 1) * 128 + (((og >> 1) ^ swz(row0 + 1)) << 4) + (og & 1) * 8) = e1;
    }
  };

  // ---- one K=16 MFMA group on LDS buffer `buf` ----
  auto mfma16 = [&](int buf, int kk) {
    const uint8_t* Ab = buf ? As1 : As0;
    const uint8_t* Bb = buf ? Bs1 : Bs0;
    const int chunk = kk * 2 + (lane >> 5);
    bf16x8 af[4], bfr[2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      af[mi] = *(const bf16x8*)(Ab + lds_off(wm * 128 + mi * 32 + (lane & 31), chunk));
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      bfr[ni] = *(const bf16x8*)(Bb + lds_off(wn * 64 + ni * 32 + (lane & 31), chunk));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
  };

  // Pipeline: tile t of A is in LDS buffer t%2 during step t; the codes of
  // tile t are loaded into register set t%2 during step t-2 and dequantized
  // into B buffer t%2 during step t-1, between that step's MFMA groups.
  // Step kt (cur = kt%2): issue A(kt+1) -> LDS cur^1 and W(kt+2) -> set cur,
  // run the MFMAs on buffer cur while dequantizing set cur^1 (tile kt+1) into
  // B buffer cur^1, wait for A(kt+1) only, barrier.
  auto step_full = [&](int kt, int cur) {
    // A's loads must be the oldest in flight: the wait at the end of the step
    // leaves only issue_W's kWLoads younger loads outstanding, so every row of
    // A(kt+1) has landed in LDS before the barrier that publishes it
    __builtin_amdgcn_sched_barrier(0);
    issue_A(kt + 1, cur ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    issue_W(kt + 2, cur);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      mfma16(cur, kk);
      dequant_quarter(cur ^ 1, cur ^ 1, kk);
    }
    __builtin_amdgcn_s_waitcnt(kWaitW);
    __syncthreads();
  };
  auto step_tail = [&](int kt, int cur) {  // last steps: no W(kt+2), maybe no A(kt+1)
    const bool more = kt + 1 < KT;
    if (more) issue_A(kt + 1, cur ^ 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      mfma16(cur, kk);
      if (more) dequant_quarter(cur ^ 1, cur ^ 1, kk);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // prologue: A(0) -> LDS 0, W(0) -> set 0, W(1) -> set 1, B(0) dequantized
  issue_A(0, 0);
  issue_W(0, 0);
  if (KT > 1) issue_W(1, 1);
  __syncthreads();  // ptab
#pragma unroll
  for (int q = 0; q < 4; ++q) dequant_quarter(0, 0, q);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  int kt = 0;
  for (; kt + 3 < KT; kt += 2) {  // both steps of the pair have kt+2 < KT
    step_full(kt, 0);
    step_full(kt + 1, 1);
  }
  // at most three steps remain; kt is even here
  if (kt + 2 < KT) {
    step_full(kt, 0);
    step_tail(kt + 1, 1);
    step_tail(kt + 2, 0);
  } else {
    if (kt < KT) step_tail(kt, 0);
    if (kt + 1 < KT) step_tail(kt + 1, 1);
  }

  // ---- adapter tail: R extra K columns from A2 [M][R] and B2 [N][R] ----
  if (p.R > 0) {
    const __amdgpu_buffer_rsrc_t a2 = make_rsrc(p.A2 + m0 * p.R, (uint32_t)(arows * p.R * 2));
    const int nrows = (N - n0) < GBN ? (N - n0) : GBN;
    const __amdgpu_buffer_rsrc_t b2 = make_rsrc(p.B2 + (int64_t)n0 * p.R, (uint32_t)(nrows * p.R * 2));
    for (int c0 = 0; c0 < p.R; c0 += GBK) {
      const int width = min(GBK, p.R - c0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = (tid >> 3) + 32 * i;
        const int kc = tid & 7;
        const uint32_t off = kc * 8 < width ? (uint32_t)((r * p.R + c0 + kc * 8) * 2) : kOOB;
        *(u32x4*)(As0 + lds_off(r, kc)) = __builtin_amdgcn_raw_buffer_load_b128(a2, off, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = tid >> 1;
        const int kc = (tid & 1) * 4 + j;
        const uint32_t off = kc * 8 < width ? (uint32_t)((r * p.R + c0 + kc * 8) * 2) : kOOB;
        *(u32x4*)(Bs0 + lds_off(r, kc)) = __builtin_amdgcn_raw_buffer_load_b128(b2, off, 0, 0);
      }
      __syncthreads();
      for (int kk = 0; kk < (width >> 4); ++kk) mfma16(0, kk);
      __syncthreads();
    }
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
  p.nblocks = (int64_t)N * K / 64;
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
