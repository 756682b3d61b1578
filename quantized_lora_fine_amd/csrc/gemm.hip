// Fused NF4-dequant bf16 MFMA GEMM for the QLoRA linear (gfx950).
//
//   C[M][N] = A[M][K] * B[N][K]^T  +  A2[M][R] * B2[N][R]^T      (fp32 accumulate)
//
// Forward  (MODE_FWD): A = X [M][h], B = w_hat(W_st) with W_st [o][h]
//                      (N = o, K = h), tail A2 = s*T [M][R], B2 = L2^T [o][R]
//                      or L2 as stored, [R][o] (b2kn > 0).
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
// Tiling: 256 x 128 output tile per 512-thread workgroup, K step 64 (one NF4
// block per W row per step), three LDS buffers each for A and the
// dequantized B.  The eight wave64s split into two roles:
//   * waves 0..3 (consumers) only read MFMA fragments from LDS and issue
//     v_mfma_f32_32x32x16_bf16; they sit 2 x 2 over the tile, 128 x 64 each
//     (4 x 2 accumulators), and read the next K=16 group's fragments while the
//     current group's MFMAs run;
//   * waves 4..7 (producers) copy A (X or dY) from global memory straight into
//     LDS with buffer_load_dwordx4 ... lds two K steps ahead, fetch W codes and
//     scales into registers three steps ahead, and dequantize the codes into
//     the B buffer two steps ahead.  Their VALU work runs on the other wave
//     slot of each SIMD, beside the consumers' MFMAs, instead of inside the
//     MFMA instruction stream.
//   One barrier per K step publishes tile s+2 and retires tile s-1, whose
//   buffer is the next one written.  Rows past M read as zero through the
//   buffer descriptor's range check, so the loop has no branches.
//   * dequant: each code byte (two NF4 codes) indexes a 256-entry LDS table of
//     fp32 value pairs; the pair is multiplied by the block scale and packed to
//     bf16 with v_cvt_pk_bf16_f32 (round to nearest even), exactly the bf16 of
//     the fp32 dequantized weight.
//   * LDS rows are 128 B (64 bf16) in 8 chunks of 16 B with an XOR swizzle so
//     that the 16-byte MFMA fragment reads are bank-conflict free.
//   * Workgroup ids are remapped so that the tiles running together on one XCD
//     (workgroups are dealt to the 8 XCDs round-robin) are consecutive in a
//     tile order that takes two row panels at a time, column by column.  The 32
//     tiles an XCD runs at once then share 2 panels of A and 16 column tiles of
//     codes, whose K steps its L2 serves to all of them: 20 % fewer bytes from
//     memory than one panel with 32 column tiles, whose codes every XCD would
//     read in full.  A group's panels are read again for each batch of 16
//     column tiles, so the 16 panels the XCDs hold at once must stay in the
//     256 MB Infinity Cache: for K > 16384 (panels over 8 MB) the order takes
//     one panel at a time.
//   * The adapter columns (R <= 64) are multiplied first: each consumer wave
//     loads its tail fragments straight into registers while the producers
//     dequantize the first tiles.  The bf16 result tile goes through LDS so
//     that every wave stores whole 128-byte lines.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace nf4k {

constexpr int GBM = 256;
constexpr int GBN = 128;
constexpr int GBK = 64;
constexpr int GNT = 512;
constexpr uint32_t kRsrcFlags = 0x00020000u;  // raw buffer, gfx9-family dword3
constexpr uint32_t kOOB = 0x80000000u;        // an offset past every buffer's range

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* Wb;  // bf16 weight [o][h] (SRC == kSrcBF16)
  const uint8_t* codes;
  const void* absmax;
  const float* dqs;
  const uint8_t* codes2;  // residual (second-stage) NF4 tensor, same layout (RES)
  const void* absmax2;
  const float* dqs2;
  const uint16_t* A2;
  const uint16_t* B2;
  uint16_t* C;
  int64_t M;
  int N;
  int K;
  int R;     // tail width, a multiple of 16 (0 = no tail)
  int b2kn;  // 0: B2 is [N][R]; > 0: B2 is [R][N] with its first b2kn rows present
  int tiles_n;
  int group_m;  // row panels per group of the tile order (1 or 2)
  int64_t nblocks;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 3); }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }
// Input-grad B tile kept as W is stored, [k][n]: 64 rows of 128 bf16 (256 B, 16
// slots of 16 B).  Slot L of row k sits at 4*((L/4) ^ (k%4)) + ((L%4) ^ (k%4)):
// the 16 lanes of a transposing read (4 rows x 32 B) and of the producer's
// 16-byte writes (4 rows x 4 slots) then fall on distinct banks.
__device__ __forceinline__ int lds_off_kn(int k, int slot) {
  const int x = k & 3;
  return k * 256 + ((((slot >> 2) ^ x) << 2 | ((slot & 3) ^ x)) << 4);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcFlags);
}

template <int MODE, int SRC, bool RES>
__global__ __launch_bounds__(GNT) void k_nf4_gemm(GemmArgs p, NF4Consts cst) {
  constexpr bool DQ = SRC == kSrcNF4DQ;
  constexpr bool BF = SRC == kSrcBF16;
  // three buffers each for A and the dequantized B: tile t lives in buffer t%3
  // the codebook pair table is placed first in LDS (its alignment sorts it
  // ahead of the tiles), so its reads carry the address in the 16-bit offset
  // field instead of adding a base register per lookup
  __shared__ __attribute__((aligned(1024))) float2 ptab[256];
  __shared__ __attribute__((aligned(16))) uint8_t As0[GBM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t As1[GBM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t As2[GBM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Bs0[GBN * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Bs1[GBN * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Bs2[GBN * 128];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7, wave-uniform (scalar)
  const bool producer = wave >= 4;      // waves 4..7 load and dequantize, waves 0..3 multiply
  const int ptid = tid - 256;           // producer thread id 0..255
  const int wm = wave & 1;              // consumer wave tile (128 x 64)
  const int wn = (wave >> 1) & 1;

  int lid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) lid = (lid & 7) * (nwg >> 3) + (lid >> 3);
  // groups of group_m row panels (fewer in a last group), column by column
  const int tiles_m = (int)((p.M + GBM - 1) / GBM);
  const int G = p.group_m;
  const int grp = lid / (G * p.tiles_n);
  const int gm = min(G, tiles_m - G * grp);
  const int gidx = lid - G * grp * p.tiles_n;
  const int tm = G * grp + gidx % gm;
  const int tn = gidx / gm;
  const int64_t m0 = (int64_t)tm * GBM;
  const int n0 = tn * GBN;
  const int64_t M = p.M;
  const int N = p.N;
  const int K = p.K;
  const int KT = K / GBK;
  const int64_t arows = (M - m0) < GBM ? (M - m0) : GBM;

  if (tid < 256) ptab[tid] = make_float2(cst.table[tid & 15], cst.table[tid >> 4]);

  auto abuf = [&](int b) -> uint8_t* { return b == 0 ? As0 : b == 1 ? As1 : As2; };
  auto bbuf = [&](int b) -> uint8_t* { return b == 0 ? Bs0 : b == 1 ? Bs1 : Bs2; };

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Input grad (and a k-major tail): B fragments come from the [k][n] tile through
  // ds_read_b64_tr_b16.
  // In each group of 16 lanes, lane 4e+q points at row k0+e, columns nb+4q..+3,
  // and lane j receives column nb+j of rows k0..k0+3; two reads (k0 and k0+4)
  // give the 8 consecutive k of the MFMA operand.
  uint32_t b_off[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    const int nb = wn * 64 + ni * 32 + 16 * (g & 1);
    b_off[ni] = (uint32_t)(lds_off_kn(8 * (g >> 1) + e, (nb >> 3) + (q >> 1)) + 8 * (q & 1));
  }
  // ---- adapter tail: R extra K columns from A2 [M][R] and B2 ([N][R], or [R][N]
  // when b2kn > 0), in chunks of at most 64: each thread loads 4 A2 pieces and
  // 2 B2 pieces of 16 bytes, stores them in the A / B tile layouts, and the
  // consumer waves multiply them like a K step (R > 64, after the main loop).
  // With R <= 64 each consumer wave instead loads its own MFMA fragments straight
  // into registers during the prologue (tail_frags) and multiplies them while the
  // producers dequantize the first tiles.
  const int tail_nrows = (N - n0) < GBN ? (N - n0) : GBN;
  const __amdgpu_buffer_rsrc_t a2r = make_rsrc(p.A2 + m0 * p.R, (uint32_t)(arows * p.R * 2));
  const __amdgpu_buffer_rsrc_t b2r = p.b2kn ? make_rsrc(p.B2, (uint32_t)((int64_t)p.b2kn * N * 2))
                                            : make_rsrc(p.B2 + (int64_t)n0 * p.R, (uint32_t)(tail_nrows * p.R * 2));
  auto tail_load = [&](int c0, u32x4 (&ta)[4], u32x4 (&tb)[2]) {
    const int width = min(GBK, p.R - c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 64 * i;
      const int kc = tid & 7;
      const uint32_t off = kc * 8 < width ? (uint32_t)((r * p.R + c0 + kc * 8) * 2) : kOOB;
      ta[i] = __builtin_amdgcn_raw_buffer_load_b128(a2r, off, 0, 0);
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      uint32_t off;
      if (p.b2kn) {
        // k-major B2: 64 tail rows x 128 columns into the [k][n] layout
        const int e = tid + 512 * jj;
        const int kr = e >> 4, slot = e & 15;
        const bool ok = kr < width && n0 + slot * 8 < N;
        off = ok ? (uint32_t)(((int64_t)(c0 + kr) * N + n0 + slot * 8) * 2) : kOOB;
      } else {
        const int r = tid >> 2;
        const int kc = (tid & 3) * 2 + jj;
        off = kc * 8 < width ? (uint32_t)((r * p.R + c0 + kc * 8) * 2) : kOOB;
      }
      tb[jj] = __builtin_amdgcn_raw_buffer_load_b128(b2r, off, 0, 0);
    }
  };
  auto tail_store = [&](uint8_t* Ab, uint8_t* Bb, const u32x4 (&ta)[4], const u32x4 (&tb)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(Ab + lds_off((tid >> 3) + 64 * i, tid & 7)) = ta[i];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      if (p.b2kn) {
        const int e = tid + 512 * jj;
        *(u32x4*)(Bb + lds_off_kn(e >> 4, e & 15)) = tb[jj];
      } else {
        *(u32x4*)(Bb + lds_off(tid >> 2, (tid & 3) * 2 + jj)) = tb[jj];
      }
    }
  };
  // fragments of K16 group kk of the tail for this consumer wave: A2 rows
  // wm*128 + mi*32 + lane%32 and B2 rows (or k-major columns) wn*64 + ni*32 + lane%32,
  // 8 consecutive k from 8*(2*kk + lane/32); rows past M or the tile read zero
  // through the ranges, columns past N are never stored
  auto tail_frags = [&](int kk, bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {
    const int k0 = 16 * kk + 8 * (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int row = wm * 128 + mi * 32 + (lane & 31);
      fa[mi] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(a2r, (uint32_t)((row * p.R + k0) * 2), 0, 0));
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      if (p.b2kn) {
        const uint32_t n = (uint32_t)(n0 + wn * 64 + ni * 32 + (lane & 31));
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(b2r, ((uint32_t)(k0 + 2 * j) * (uint32_t)N + n) * 2, 0, 0);
          const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(b2r, ((uint32_t)(k0 + 2 * j + 1) * (uint32_t)N + n) * 2, 0, 0);
          v[j] = lo | (hi << 16);
        }
        fb[ni] = __builtin_bit_cast(bf16x8, v);
      } else {
        const int row = wn * 64 + ni * 32 + (lane & 31);
        fb[ni] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(b2r, (uint32_t)((row * p.R + k0) * 2), 0, 0));
      }
    }
  };
  auto tail_mma = [&](const uint8_t* Ab, const uint8_t* Bb, int width) {
    for (int kk = 0; kk < (width >> 4); ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      bf16x8 fa[4], fb[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) fa[mi] = *(const bf16x8*)(Ab + lds_off(wm * 128 + mi * 32 + (lane & 31), chunk));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        if (p.b2kn) fb[ni] = lds_tr8(const_cast<uint8_t*>(Bb) + kk * 4096 + b_off[ni], 256);
        else fb[ni] = *(const bf16x8*)(Bb + lds_off(wn * 64 + ni * 32 + (lane & 31), chunk));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ni], fa[mi], acc[mi][ni], 0, 0, 0);
    }
  };
  const bool early_tail = p.R > 0 && p.R <= GBK;

  if (producer) {
    // ================= producer waves =================
    const int pw = wave - 4;
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.A + m0 * K, (uint32_t)(arows * K * 2));
    uint32_t a_voff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (pw * 8 + i) * 8 + (lane >> 3);
      a_voff[i] = (uint32_t)(r * K * 2 + (((lane & 7) ^ swz(r)) << 4));
    }
    // The step's column offset goes in the scalar soffset field (no VALU add per
    // copy). Rows past M still read zero through the range check on voffset;
    // steps past K are not issued at all (callers check kt < KT).
    auto issue_A = [&](int kt, int b) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint8_t* dst = abuf(b) + (pw * 8 + i) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)dst, 16, a_voff[i], kt * 128, 0, 0);
      }
    };
    // Each producer thread owns 32 consecutive weights of one W row per K step:
    //   FWD: B row n = ptid/2 (W row n0+n), K columns 32*(ptid%2) .. +32 of the step;
    //   DX : step row kr = 16*pw + lane/4 (W row 64*kt + kr), columns n0 + 32*(lane%4) .. +32.
    // Either way that is one 16-byte load of codes (64 bytes of bf16) and one block
    // scale, dequantized into four 16-byte chunks of the B tile.
    const int kr = pw * 16 + (lane >> 2);
    const int cq = lane & 3;
    __amdgpu_buffer_rsrc_t c_rsrc;
    uint32_t c_voff, s_voff = 0, c_step, s_step = 0;
    if constexpr (MODE == MODE_FWD) {
      const int n = ptid >> 1;
      const int nrows = (N - n0) < GBN ? (N - n0) : GBN;
      if constexpr (BF) {
        c_rsrc = make_rsrc(p.Wb + (int64_t)n0 * K, (uint32_t)((int64_t)nrows * K * 2));
        c_voff = (uint32_t)(n * K * 2 + (ptid & 1) * 64);
        c_step = 128;
      } else {
        c_rsrc = make_rsrc(p.codes + (int64_t)n0 * (K >> 1), (uint32_t)((int64_t)nrows * (K >> 1)));
        c_voff = (uint32_t)(n * (K >> 1) + (ptid & 1) * 16);
        c_step = 32;
        s_voff = (uint32_t)(n0 + n) * (uint32_t)(K >> 6);
        s_step = 1;
      }
    } else {
      const bool ok = n0 + cq * 32 < N;  // N is a multiple of 64: a chunk is all in or all out
      if constexpr (BF) {
        c_rsrc = make_rsrc(p.Wb, (uint32_t)((int64_t)K * N * 2));
        c_voff = ok ? (uint32_t)((kr * N + n0 + cq * 32) * 2) : kOOB;
        c_step = 128u * (uint32_t)N;
      } else {
        c_rsrc = make_rsrc(p.codes, (uint32_t)(p.nblocks * 32));
        c_voff = ok ? (uint32_t)(kr * (N >> 1) + ((n0 + cq * 32) >> 1)) : kOOB;
        c_step = 32u * (uint32_t)N;
        s_voff = ok ? (uint32_t)(kr * (N >> 6) + ((n0 + cq * 32) >> 6)) : kOOB;
        s_step = (uint32_t)N;
      }
    }
    // LDS byte offsets of the thread's four 16-byte chunks in a B buffer
    uint32_t w_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (MODE == MODE_FWD) w_off[q] = (uint32_t)lds_off(ptid >> 1, (ptid & 1) * 4 + q);
      else w_off[q] = (uint32_t)lds_off_kn(kr, cq * 4 + q);
    }
    const __amdgpu_buffer_rsrc_t s_rsrc = make_rsrc(p.absmax, (uint32_t)(p.nblocks * (DQ ? 1 : 4)));
    const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(p.dqs, (uint32_t)(DQ ? ((p.nblocks + 255) / 256) * 4 : 0));
    // the residual stage: same offsets into its own buffers
    __amdgpu_buffer_rsrc_t c2_rsrc = c_rsrc, s2_rsrc = s_rsrc, q2_rsrc = q_rsrc;
    if constexpr (RES) {
      if constexpr (MODE == MODE_FWD) {
        const int nrows = (N - n0) < GBN ? (N - n0) : GBN;
        c2_rsrc = make_rsrc(p.codes2 + (int64_t)n0 * (K >> 1), (uint32_t)((int64_t)nrows * (K >> 1)));
      } else {
        c2_rsrc = make_rsrc(p.codes2, (uint32_t)(p.nblocks * 32));
      }
      s2_rsrc = make_rsrc(p.absmax2, (uint32_t)(p.nblocks * (DQ ? 1 : 4)));
      q2_rsrc = make_rsrc(p.dqs2, (uint32_t)(DQ ? ((p.nblocks + 255) / 256) * 4 : 0));
    }

    u32x4 creg[2], creg2[2];
    uint32_t sraw[2], sraw2[2];
    float sstep[2], sstep2[2];
    auto load_scale = [&](uint32_t blk, int set) {
      if constexpr (DQ) {
        sraw[set] = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, blk, 0, 0);
        sstep[set] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(q_rsrc, (blk >> 8) * 4, 0, 0));
      } else {
        sraw[set] = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, blk * 4, 0, 0);
      }
    };
    auto load_scale2 = [&](uint32_t blk, int set) {
      if constexpr (DQ) {
        sraw2[set] = __builtin_amdgcn_raw_buffer_load_b8(s2_rsrc, blk, 0, 0);
        sstep2[set] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(q2_rsrc, (blk >> 8) * 4, 0, 0));
      } else {
        sraw2[set] = __builtin_amdgcn_raw_buffer_load_b32(s2_rsrc, blk * 4, 0, 0);
      }
    };
    auto scale = [&](int set) -> float {
      if constexpr (DQ) return (float)sraw[set] * sstep[set];
      else return __builtin_bit_cast(float, sraw[set]);
    };
    auto scale2 = [&](int set) -> float {
      if constexpr (DQ) return (float)sraw2[set] * sstep2[set];
      else return __builtin_bit_cast(float, sraw2[set]);
    };
    // dequantized weight of one code: fl32(t * sc), or with the residual stage
    // fl32(fl32(t * sc) + fl32(t2 * sc2)) (no fused multiply-add)
    auto wval = [&](float t, float sc, float t2, float sc2) -> float {
      if constexpr (RES) return __fadd_rn(__fmul_rn(t, sc), __fmul_rn(t2, sc2));
      else return t * sc;
    };
    u32x4 wreg[2][4];  // bf16 weight chunks (SRC == kSrcBF16)
    // codes (or bf16 W) with the step offset in soffset, as for X; only for kt < KT
    auto issue_W = [&](int kt, int set) {
      const int cs = (int)((uint32_t)kt * c_step);
      if constexpr (BF) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          wreg[set][q] = __builtin_amdgcn_raw_buffer_load_b128(c_rsrc, c_voff + q * 16, cs, 0);
      } else {
        const uint32_t so = s_voff + (uint32_t)kt * s_step;
        creg[set] = __builtin_amdgcn_raw_buffer_load_b128(c_rsrc, c_voff, cs, 0);
        load_scale(so, set);
        if constexpr (RES) {
          creg2[set] = __builtin_amdgcn_raw_buffer_load_b128(c2_rsrc, c_voff, cs, 0);
          load_scale2(so, set);
        }
      }
    };
    constexpr int kWLoads = BF ? 4 : (DQ ? 3 : 2) * (RES ? 2 : 1);
    constexpr int kWaitW = (kWLoads & 15) | ((kWLoads >> 4) << 14) | (0x7 << 4) | (0xF << 8);
    auto dequant = [&](int set, int b) {
      uint8_t* dst = bbuf(b);
      if constexpr (BF) {
        // bf16 source: the 4 chunks go to the tile as they are
#pragma unroll
        for (int q = 0; q < 4; ++q) *(u32x4*)(dst + w_off[q]) = wreg[set][q];
      } else {
        // all table reads first: one LDS round trip per step, not one per 16-byte chunk
        float2 t[4][4], t2[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int bq = 0; bq < 4; ++bq) {
            t[q][bq] = ptab[(creg[set][q] >> (8 * bq)) & 0xFFu];
            if constexpr (RES) t2[q][bq] = ptab[(creg2[set][q] >> (8 * bq)) & 0xFFu];
            else t2[q][bq] = make_float2(0.f, 0.f);
          }
        const float sc = scale(set);
        const float sc2 = RES ? scale2(set) : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x4 o;
#pragma unroll
          for (int bq = 0; bq < 4; ++bq)
            o[bq] = pack_bf16x2(wval(t[q][bq].x, sc, t2[q][bq].x, sc2), wval(t[q][bq].y, sc, t2[q][bq].y, sc2));
          *(u32x4*)(dst + w_off[q]) = o;
        }
      }
    };
    // prologue: tiles 0 and 1 into buffers 0 and 1; W(2) into set 0
    issue_A(0, 0);
    if (KT > 1) issue_A(1, 1);
    issue_W(0, 0);
    if (KT > 1) issue_W(1, 1);
    __syncthreads();  // (1) ptab
    dequant(0, 0);
    if (KT > 1) dequant(1, 1);
    if (KT > 2) {
      issue_W(2, 0);
      __builtin_amdgcn_s_waitcnt(kWaitW);  // all but W(2): the X copies have landed
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();  // (2) tiles 0, 1 published
    // step s: produce tile s+2 (A DMA into buffer (s+2)%3, dequant from set s%2),
    // fetch the codes of tile s+3 into set (s+1)%2, then the step's barrier.
    // Buffer (s+2)%3 held tile s-1, fully consumed before the previous barrier.
    // Near the end, tiles past K are neither loaded nor dequantized; a step that
    // issues no codes waits for every load (the fixed count assumes W was last).
    // FULL steps (s + 3 < KT) skip the checks.
    auto pstep = [&](int s, int j, auto full) {
      __builtin_amdgcn_sched_barrier(0);
      if (full || s + 2 < KT) issue_A(s + 2, (j + 2) % 3);
      __builtin_amdgcn_sched_barrier(0);
      if (full || s + 3 < KT) issue_W(s + 3, (j + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      if (full || s + 2 < KT) dequant(j & 1, (j + 2) % 3);
      if (full || s + 3 < KT) __builtin_amdgcn_s_waitcnt(kWaitW);  // all but W(s+3): X of tile s+2 landed
      else __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    constexpr std::true_type kFull{};
    constexpr std::false_type kTail{};
    int s = 0;
    for (; s + 9 <= KT; s += 6) {
      pstep(s, 0, kFull); pstep(s + 1, 1, kFull); pstep(s + 2, 2, kFull);
      pstep(s + 3, 3, kFull); pstep(s + 4, 4, kFull); pstep(s + 5, 5, kFull);
    }
    // at most 8 steps remain; j keeps counting modulo 6
    if (s < KT) pstep(s, 0, kTail);
    if (s + 1 < KT) pstep(s + 1, 1, kTail);
    if (s + 2 < KT) pstep(s + 2, 2, kTail);
    if (s + 3 < KT) pstep(s + 3, 3, kTail);
    if (s + 4 < KT) pstep(s + 4, 4, kTail);
    if (s + 5 < KT) pstep(s + 5, 5, kTail);
    if (s + 6 < KT) pstep(s + 6, 0, kTail);
    if (s + 7 < KT) pstep(s + 7, 1, kTail);
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    // ================= consumer waves: fragment reads and MFMAs only =================
    struct Frags {
      bf16x8 a[4], b[2];
    };
    auto load_frags = [&](int b, int kk, Frags& f) {
      const uint8_t* Ab = abuf(b);
      const uint8_t* Bb = bbuf(b);
      const int chunk = kk * 2 + (lane >> 5);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        f.a[mi] = *(const bf16x8*)(Ab + lds_off(wm * 128 + mi * 32 + (lane & 31), chunk));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        if constexpr (MODE == MODE_FWD) {
          f.b[ni] = *(const bf16x8*)(Bb + lds_off(wn * 64 + ni * 32 + (lane & 31), chunk));
        } else {
          f.b[ni] = lds_tr8(const_cast<uint8_t*>(Bb) + kk * 4096 + b_off[ni], 256);
        }
      }
    };
    auto mma = [&](const Frags& f) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0);
    };
    constexpr int kReads = MODE == MODE_FWD ? 6 : 8;  // LDS reads per K16 group
    auto interleave = [&]() {
#pragma unroll
      for (int i = 0; i < kReads; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one fragment read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
      if constexpr (kReads < 8) __builtin_amdgcn_sched_group_barrier(0x008, 8 - kReads, 0);
    };
    Frags f0, f1;
    {
      // the adapter tail (R <= 64): group 0's loads go out before barrier (1),
      // its MFMAs (and the later groups') run before barrier (2)
      bf16x8 tfa[4], tfb[2];
      if (early_tail) tail_frags(0, tfa, tfb);
      __syncthreads();  // (1)
      if (early_tail) {
        for (int kk = 0;;) {
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfb[ni], tfa[mi], acc[mi][ni], 0, 0, 0);
          if (++kk >= (p.R >> 4)) break;
          tail_frags(kk, tfa, tfb);
        }
      }
    }
    __syncthreads();  // (2)
    load_frags(0, 0, f0);
    // step s: tile s (buffer s%3) is published and f0 holds its first K16
    // fragments; the next group's reads are issued during the current group's
    // MFMAs, the last one being the first group of tile s+1 (published one
    // step earlier), so no step starts by waiting on LDS.
    auto cstep = [&](int j) {
      const int b = j % 3, bn = (j + 1) % 3;
      load_frags(b, 1, f1);
      mma(f0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      load_frags(b, 2, f0);
      mma(f1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      load_frags(b, 3, f1);
      mma(f0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      load_frags(bn, 0, f0);
      mma(f1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    };
    int s = 0;
    for (; s + 6 <= KT; s += 6) {
      cstep(0); cstep(1); cstep(2); cstep(3); cstep(4); cstep(5);
    }
    if (s < KT) cstep(0);
    if (s + 1 < KT) cstep(1);
    if (s + 2 < KT) cstep(2);
    if (s + 3 < KT) cstep(3);
    if (s + 4 < KT) cstep(4);
  }
  __syncthreads();

  // ---- adapter tail for R > 64: chunks through buffers 0 after the main loop ----
  if (p.R > 0 && !early_tail) {
    for (int c0 = 0; c0 < p.R; c0 += GBK) {
      u32x4 xa[4], xb[2];
      tail_load(c0, xa, xb);
      tail_store(As0, Bs0, xa, xb);
      __syncthreads();
      if (!producer) tail_mma(As0, Bs0, min(GBK, p.R - c0));
      __syncthreads();
    }
  }

  // ---- epilogue: D[n][m], lane holds m = l%32, n = 8*(v/4) + 4*(l/32) + v%4.  The
  // consumers write the bf16 tile to LDS (A buffer 0: rows 0..127, buffer 1: rows
  // 128..255; 256-byte rows whose 16-byte chunks are XOR-swizzled by row % 16),
  // then all waves store it as contiguous 16-byte pieces, 4 rows per wave store. ----
  if (!producer) {
    uint8_t* stg = wm == 0 ? As0 : As1;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int row = mi * 32 + (lane & 31);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int col = wn * 64 + ni * 32 + 8 * gg + 4 * (lane >> 5);
          uint2 o;
          o.x = pack_bf16x2(acc[mi][ni][4 * gg + 0], acc[mi][ni][4 * gg + 1]);
          o.y = pack_bf16x2(acc[mi][ni][4 * gg + 2], acc[mi][ni][4 * gg + 3]);
          *(uint2*)(stg + row * 256 + (((col >> 3) ^ (row & 15)) << 4) + ((col >> 2) & 1) * 8) = o;
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int e = tid + 512 * it;
    const int row = e >> 4, piece = e & 15;
    const int64_t m = m0 + row;
    const int n = n0 + piece * 8;
    if (m < M && n < N) {
      const int r = row & 127;
      const uint8_t* stg = row < 128 ? As0 : As1;
      *(u32x4*)(p.C + m * N + n) = *(const u32x4*)(stg + r * 256 + ((piece ^ (r & 15)) << 4));
    }
  }
}

hipError_t launch_nf4_gemm(int mode, int src, const uint16_t* A, const uint16_t* Wb, const uint8_t* codes,
                           const void* absmax, const float* dqs, const uint8_t* codes2, const void* absmax2,
                           const float* dqs2, const uint16_t* A2, const uint16_t* B2, int R, int b2kn, uint16_t* C,
                           int64_t M, int N, int K, const NF4Consts& c, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmArgs p;
  p.A = A;
  p.Wb = Wb;
  p.codes = codes;
  p.absmax = absmax;
  p.dqs = dqs;
  p.codes2 = codes2;
  p.absmax2 = absmax2;
  p.dqs2 = dqs2;
  p.A2 = A2;
  p.B2 = B2;
  p.C = C;
  p.M = M;
  p.N = N;
  p.K = K;
  p.R = R;
  p.b2kn = R > 0 ? b2kn : 0;
  p.nblocks = (int64_t)N * K / 64;
  const int64_t tiles_m = (M + GBM - 1) / GBM;
  p.tiles_n = (N + GBN - 1) / GBN;
  p.group_m = gemm_group_m(K);  // see the tile order in the header
  const bool res = codes2 != nullptr && src != kSrcBF16;
  // A launch holds at most 2^32 - 1 work-items (GNT per tile).  Each row of C
  // depends only on its own rows of A and A2, so a product with more tiles runs
  // as launches over consecutive ranges of row panels.
  static_assert(GNT == 512, "gemm_launch_panels counts 512 work-items per tile");
  const int64_t panels = gemm_launch_panels(p.tiles_n);
  for (int64_t t0 = 0; t0 < tiles_m; t0 += panels) {
    const int64_t m0 = t0 * GBM;
    const int64_t tm = std::min(panels, tiles_m - t0);
    GemmArgs q = p;
    q.A = A + m0 * K;
    q.A2 = A2 ? A2 + m0 * R : nullptr;
    q.C = C + m0 * N;
    q.M = std::min(tm * GBM, M - m0);
    const dim3 gr((unsigned)(tm * p.tiles_n)), bl(GNT);
#define NF4K_GEMM(MD, SR, RS) hipLaunchKernelGGL((k_nf4_gemm<MD, SR, RS>), gr, bl, 0, st, q, c)
#define NF4K_GEMM_SRC(MD)                                                                      \
  if (src == kSrcBF16) NF4K_GEMM(MD, kSrcBF16, false);                                         \
  else if (src == kSrcNF4DQ) { if (res) NF4K_GEMM(MD, kSrcNF4DQ, true); else NF4K_GEMM(MD, kSrcNF4DQ, false); } \
  else { if (res) NF4K_GEMM(MD, kSrcNF4, true); else NF4K_GEMM(MD, kSrcNF4, false); }
    if (mode == MODE_FWD) {
      NF4K_GEMM_SRC(MODE_FWD)
    } else {
      NF4K_GEMM_SRC(MODE_DX)
    }
#undef NF4K_GEMM_SRC
#undef NF4K_GEMM
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nf4k
