// Merge of a trained adapter into the frozen base (gfx950).
//
// "LoRA: Fine-tuning a model by learning a small update", section "Serving
// models and switching tasks": the learned update is added to the pretrained
// matrix once (W_merged = W0 + (alpha/r) B A), after which the layer is an
// ordinary dense one.  In the storage layout used here (W [o][h], Y = X W^T +
// s X L1 L2) that is
//     W'[n][k] = base[n][k] + s * sum_j L2[j][n] * L1[k][j].
// "Lesson 17. What QLoRA Actually Costs" merges an adapter trained against a
// 4-bit base into the full-precision base and quantises afterwards if needed:
// the base is the fp32 W when the caller has it, else the NF4 weight
// dequantized exactly as nf4_dequantize does; re-quantizing the fp32 result is
// an nf4_quantize call.
//
// One workgroup (256 threads) owns 16 rows x 256 columns of W'.  Per chunk of
// 64 adapter columns it stages L1^T [j][k] (bf16, transposed, rows padded so
// the 16-byte reads are conflict free) and L2 [j][n] (fp32) in LDS; thread t
// accumulates columns 8*(t%32) .. +7 of rows t/32 and t/32 + 8 with fp32 FMAs,
// then adds the base (read once from HBM) and writes the row segment with
// 16/32-byte stores.  HBM-bound for small r (r FMAs per weight against 4-6
// bytes moved).
#include "common.hpp"
#include "launch.hpp"

namespace nf4k {

constexpr int MG_COLS = 256;  // columns per workgroup
constexpr int MG_ROWS = 16;   // rows per workgroup
constexpr int MG_RC = 64;     // adapter columns per LDS chunk
constexpr int MG_LDT = MG_COLS + 8;

// BASE: 0 fp32 W, 1 NF4 (fp32 absmax), 2 NF4 (8-bit scales); RES: NF4 base with a residual stage
template <int BASE, bool OUT_BF16, bool RES>
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ W, const uint8_t* __restrict__ codes,
                                               const void* __restrict__ absmax, const float* __restrict__ dqs,
                                               const uint8_t* __restrict__ codes2, const void* __restrict__ absmax2,
                                               const float* __restrict__ dqs2,
                                               const uint16_t* __restrict__ L1, const uint16_t* __restrict__ L2,
                                               int r, float s, int64_t rows, int64_t cols, void* __restrict__ out,
                                               NF4Consts cst) {
  __shared__ __attribute__((aligned(16))) uint16_t l1t[MG_RC * MG_LDT];
  __shared__ float l2s[MG_RC * MG_ROWS];
  __shared__ float tab[16];
  const int t = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * MG_COLS;
  const int64_t n0 = (int64_t)blockIdx.y * MG_ROWS;
  const int kl = (t & 31) * 8;
  const int rl0 = t >> 5, rl1 = rl0 + 8;
  if (t < 16) tab[t] = cst.table[t];

  float acc0[8], acc1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc0[e] = acc1[e] = 0.f;

  for (int j0 = 0; j0 < r; j0 += MG_RC) {
    const int jn = min(MG_RC, r - j0);
    __syncthreads();  // previous chunk fully read
    if ((r & 7) == 0) {
      // 8 adapter columns per 16-byte load (L1 rows are 16-byte aligned when r % 8 == 0)
      const int j8n = jn >> 3;
      for (int e = t; e < j8n * MG_COLS; e += 256) {
        const int j8 = e % j8n, kk = e / j8n;
        const int64_t k = k0 + kk;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (k < cols) v = *(const u32x4*)(L1 + k * r + j0 + j8 * 8);
#pragma unroll
        for (int q = 0; q < 8; ++q) l1t[(j8 * 8 + q) * MG_LDT + kk] = (uint16_t)(v[q >> 1] >> (16 * (q & 1)));
      }
    } else {
      for (int e = t; e < jn * MG_COLS; e += 256) {
        const int jj = e % jn, kk = e / jn;  // consecutive threads walk j: contiguous L1 reads
        const int64_t k = k0 + kk;
        l1t[jj * MG_LDT + kk] = k < cols ? L1[k * r + j0 + jj] : (uint16_t)0;
      }
    }
    for (int e = t; e < jn * MG_ROWS; e += 256) {
      const int jj = e / MG_ROWS, nl = e % MG_ROWS;
      const int64_t n = n0 + nl;
      l2s[e] = n < rows ? bf16_to_f32(L2[(int64_t)(j0 + jj) * rows + n]) : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < jn; ++jj) {
      const u32x4 b = *(const u32x4*)&l1t[jj * MG_LDT + kl];
      const float a0 = l2s[jj * MG_ROWS + rl0], a1 = l2s[jj * MG_ROWS + rl1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float bv = bf16_to_f32((uint16_t)(b[e >> 1] >> (16 * (e & 1))));
        acc0[e] = fmaf(a0, bv, acc0[e]);
        acc1[e] = fmaf(a1, bv, acc1[e]);
      }
    }
  }
  __syncthreads();  // tab[]

  const int64_t k = k0 + kl;
  if (k >= cols) return;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t n = n0 + (h ? rl1 : rl0);
    if (n >= rows) continue;
    const float* acc = h ? acc1 : acc0;
    const int64_t idx = n * cols + k;  // first of 8 weights (same NF4 block: k % 8 == 0, cols % 64 == 0)
    float base[8];
    if constexpr (BASE == 0) {
      const floatx4 u = *(const floatx4*)(W + idx), v = *(const floatx4*)(W + idx + 4);
      base[0] = u.x; base[1] = u.y; base[2] = u.z; base[3] = u.w;
      base[4] = v.x; base[5] = v.y; base[6] = v.z; base[7] = v.w;
    } else {
      const int64_t blk = idx / 64;
      auto scale = [&](const void* am, const float* dq) -> float {
        if constexpr (BASE == 2) return (float)((const uint8_t*)am)[blk] * dq[blk / 256];
        else return ((const float*)am)[blk];
      };
      const uint32_t c = *(const uint32_t*)(codes + idx / 2);
      const float sc = scale(absmax, dqs);
#pragma unroll
      for (int e = 0; e < 8; ++e) base[e] = __fmul_rn(tab[(c >> (4 * e)) & 15u], sc);
      if constexpr (RES) {
        // two-stage weight: fl32(w_hat1 + w_hat2), exactly as nf4_dequantize forms it
        const uint32_t c2 = *(const uint32_t*)(codes2 + idx / 2);
        const float sc2 = scale(absmax2, dqs2);
#pragma unroll
        for (int e = 0; e < 8; ++e) base[e] = __fadd_rn(base[e], __fmul_rn(tab[(c2 >> (4 * e)) & 15u], sc2));
      }
    }
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = base[e] + s * acc[e];
    if constexpr (OUT_BF16) {
      const u32x4 p = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                       pack_bf16x2(o[6], o[7])};
      *(u32x4*)((uint16_t*)out + idx) = p;
    } else {
      *(floatx4*)((float*)out + idx) = floatx4{o[0], o[1], o[2], o[3]};
      *(floatx4*)((float*)out + idx + 4) = floatx4{o[4], o[5], o[6], o[7]};
    }
  }
}

// MFMA variant for RP = 16*ceil(r/16) <= 64.  One workgroup (256 threads)
// owns 64 rows x 128 columns of W'.  It stages L2[:, rows] ([RP][64], rows
// padded to 144 B so a transposing read's 4 rows hit distinct banks) and
// L1[cols, :] ([128][RP]) in LDS, zero past r; each wave multiplies two 32x32
// blocks of (L1 L2)^T with v_mfma_f32_32x32x16_bf16 (bf16 products exact,
// fp32 sums), the L2 operand read transposed with ds_read_b64_tr_b16.  The
// fp32 products go through LDS so that each thread then owns 8 consecutive
// columns of a row: one code word and one block scale for the NF4 base, the
// add and one 16/32-byte store.
constexpr int MM_ROWS = 64, MM_COLS = 128, MM_L2ROW = 144, MM_ACCROW = MM_COLS + 4;

template <int BASE, bool OUT_BF16, bool RES>
__global__ __launch_bounds__(256) void k_merge_mfma(const float* __restrict__ W, const uint8_t* __restrict__ codes,
                                                    const void* __restrict__ absmax, const float* __restrict__ dqs,
                                                    const uint8_t* __restrict__ codes2,
                                                    const void* __restrict__ absmax2, const float* __restrict__ dqs2,
                                                    const uint16_t* __restrict__ L1, const uint16_t* __restrict__ L2,
                                                    int r, int RP, float s, int64_t rows, int64_t cols,
                                                    void* __restrict__ out, NF4Consts cst) {
  // the adapter slices are dead once the products are in registers: the fp32
  // product tile reuses their LDS (4 workgroups fit on a CU)
  constexpr int kSlices = 64 * MM_L2ROW + MM_COLS * 64 * 2, kAcc = MM_ROWS * MM_ACCROW * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSlices > kAcc ? kSlices : kAcc];
  uint8_t* const l2s = smem;                                   // [j][n], rows of 144 B
  uint16_t* const l1s = (uint16_t*)(smem + 64 * MM_L2ROW);     // [k][j], rows of RP
  float* const accs = (float*)smem;                            // [n][k], rows of MM_ACCROW
  __shared__ float tab[16];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int64_t n0 = (int64_t)blockIdx.y * MM_ROWS;
  const int64_t k0 = (int64_t)blockIdx.x * MM_COLS;
  if (t < 16) tab[t] = cst.table[t];
  // this thread's base data first, so its latency hides behind the staging and
  // the products: 4 segments of 8 consecutive columns (64 rows x 16 segments)
  uint32_t cw[4], cw2[4];
  float scv[4], scv2[4];
  floatx4 wv[4][2];
#pragma unroll
  for (int seg = 0; seg < 4; ++seg) {
    const int e = t + 256 * seg;
    const int64_t n = n0 + (e >> 4), k = k0 + (e & 15) * 8;
    const bool ok = n < rows && k < cols;
    const int64_t idx = ok ? n * cols + k : 0;
    if constexpr (BASE == 0) {
      wv[seg][0] = *(const floatx4*)(W + idx);
      wv[seg][1] = *(const floatx4*)(W + idx + 4);
    } else {
      const int64_t blk = idx / 64;
      auto scale = [&](const void* am, const float* dq) -> float {
        if constexpr (BASE == 2) return (float)((const uint8_t*)am)[blk] * dq[blk / 256];
        else return ((const float*)am)[blk];
      };
      cw[seg] = *(const uint32_t*)(codes + idx / 2);
      scv[seg] = scale(absmax, dqs);
      if constexpr (RES) {
        cw2[seg] = *(const uint32_t*)(codes2 + idx / 2);
        scv2[seg] = scale(absmax2, dqs2);
      }
    }
  }
  // L2 slice: RP rows x 64 columns (8 bf16 per thread-step), zero past r / rows
  for (int e = t; e < RP * 8; e += 256) {
    const int j = e >> 3, c8 = (e & 7) * 8;
    const int64_t n = n0 + c8;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (j < r) {
      if (n + 8 <= rows && ((rows & 7) == 0)) {
        v = *(const u32x4*)(L2 + (int64_t)j * rows + n);
      } else {
        uint16_t h8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) h8[q] = (n + q < rows) ? L2[(int64_t)j * rows + n + q] : (uint16_t)0;
        v = u32x4{h8[0] | ((uint32_t)h8[1] << 16), h8[2] | ((uint32_t)h8[3] << 16), h8[4] | ((uint32_t)h8[5] << 16),
                  h8[6] | ((uint32_t)h8[7] << 16)};
      }
    }
    *(u32x4*)(l2s + j * MM_L2ROW + c8 * 2) = v;
  }
  // L1 slice: 128 rows (columns of W') x RP, zero past r / cols; 16-byte pieces
  // when r % 8 == 0 (L1 rows are then 16-byte aligned)
  if ((r & 7) == 0) {
    const int P = RP / 8;
    for (int e = t; e < MM_COLS * P; e += 256) {
      const int kk = e / P, j8 = (e - kk * P) * 8;
      const int64_t k = k0 + kk;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (j8 < r && k < cols) v = *(const u32x4*)(L1 + k * r + j8);
      *(u32x4*)(l1s + kk * RP + j8) = v;
    }
  } else {
    for (int e = t; e < MM_COLS * RP; e += 256) {
      const int kk = e / RP, j = e - kk * RP;
      const int64_t k = k0 + kk;
      l1s[kk * RP + j] = (j < r && k < cols) ? L1[k * r + j] : (uint16_t)0;
    }
  }
  __syncthreads();

  // wave w: rows 32*(w/2) .. +32, columns 64*(w%2) .. +64 (two 32x32 blocks)
  const int rb = 32 * (wave >> 1), cb = 64 * (wave & 1);
  floatx16 acc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
  const int g = lane >> 4, e4 = (lane >> 2) & 3, q4 = lane & 3;
  for (int ks = 0; ks < RP; ks += 16) {
    // A operand (rows n, 8 consecutive j): transposed from the [j][n] slice
    const bf16x8 a = lds_tr8(l2s + (ks + 8 * (g >> 1) + e4) * MM_L2ROW + 2 * (rb + 16 * (g & 1) + 4 * q4), MM_L2ROW);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      // B operand (rows k, 8 consecutive j): row-major [k][j]
      const bf16x8 bk = *(const bf16x8*)(l1s + (cb + 32 * b + (lane & 31)) * RP + ks + 8 * (lane >> 5));
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bk, acc[b], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave has read its operands; the tile overwrites them
  // D[n][k]: lane holds k = lane%32 of its block, n = 8*(v/4) + 4*(lane/32) + v%4
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int n = rb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      accs[n * MM_ACCROW + cb + 32 * b + (lane & 31)] = acc[b][v];
    }
  __syncthreads();

  // thread: 8 consecutive columns of a row, 4 segments
#pragma unroll
  for (int seg = 0; seg < 4; ++seg) {
    const int e = t + 256 * seg;           // 64 rows x 16 segments of 8
    const int nl = e >> 4, kl = (e & 15) * 8;
    const int64_t n = n0 + nl, k = k0 + kl;
    if (n >= rows || k >= cols) continue;
    const int64_t idx = n * cols + k;      // first of 8 weights (one NF4 block: cols % 64 == 0)
    float base[8];
    if constexpr (BASE == 0) {
      const floatx4 u = wv[seg][0], w = wv[seg][1];
      base[0] = u.x; base[1] = u.y; base[2] = u.z; base[3] = u.w;
      base[4] = w.x; base[5] = w.y; base[6] = w.z; base[7] = w.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) base[q] = __fmul_rn(tab[(cw[seg] >> (4 * q)) & 15u], scv[seg]);
      if constexpr (RES) {
        // two-stage weight: fl32(w_hat1 + w_hat2), exactly as nf4_dequantize forms it
#pragma unroll
        for (int q = 0; q < 8; ++q) base[q] = __fadd_rn(base[q], __fmul_rn(tab[(cw2[seg] >> (4 * q)) & 15u], scv2[seg]));
      }
    }
    const floatx4 a0 = *(const floatx4*)(accs + nl * MM_ACCROW + kl);
    const floatx4 a1 = *(const floatx4*)(accs + nl * MM_ACCROW + kl + 4);
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    float o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = base[q] + s * av[q];
    if constexpr (OUT_BF16) {
      const u32x4 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                        pack_bf16x2(o[6], o[7])};
      *(u32x4*)((uint16_t*)out + idx) = pk;
    } else {
      *(floatx4*)((float*)out + idx) = floatx4{o[0], o[1], o[2], o[3]};
      *(floatx4*)((float*)out + idx + 4) = floatx4{o[4], o[5], o[6], o[7]};
    }
  }
}

hipError_t launch_merge(int base, const float* W, const uint8_t* codes, const void* absmax, const float* dqs,
                        const uint8_t* codes2, const void* absmax2, const float* dqs2, const uint16_t* L1,
                        const uint16_t* L2, int r, float s, int64_t rows, int64_t cols, bool out_bf16, void* out,
                        const NF4Consts& c, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const bool res = base != 0 && codes2 != nullptr;
  const int RP = (r + 15) / 16 * 16;
  if (RP <= 64) {
    const dim3 gm((unsigned)((cols + MM_COLS - 1) / MM_COLS), (unsigned)((rows + MM_ROWS - 1) / MM_ROWS)), bm(256);
#define NF4K_MERGE_M(B, O, R)                                                                                    \
  hipLaunchKernelGGL((k_merge_mfma<B, O, R>), gm, bm, 0, st, W, codes, absmax, dqs, codes2, absmax2, dqs2, L1, L2, \
                     r, RP, s, rows, cols, out, c)
#define NF4K_MERGE_MO(B, R) \
  if (out_bf16) NF4K_MERGE_M(B, true, R); else NF4K_MERGE_M(B, false, R);
    if (base == 0) {
      NF4K_MERGE_MO(0, false)
    } else if (base == 1) {
      if (res) { NF4K_MERGE_MO(1, true) } else { NF4K_MERGE_MO(1, false) }
    } else {
      if (res) { NF4K_MERGE_MO(2, true) } else { NF4K_MERGE_MO(2, false) }
    }
#undef NF4K_MERGE_MO
#undef NF4K_MERGE_M
    return hipGetLastError();
  }
  const dim3 gr((unsigned)((cols + MG_COLS - 1) / MG_COLS), (unsigned)((rows + MG_ROWS - 1) / MG_ROWS)), bl(256);
#define NF4K_MERGE(B, O, R)                                                                                        \
  hipLaunchKernelGGL((k_merge<B, O, R>), gr, bl, 0, st, W, codes, absmax, dqs, codes2, absmax2, dqs2, L1, L2, r, s, \
                     rows, cols, out, c)
#define NF4K_MERGE_O(B, R) \
  if (out_bf16) NF4K_MERGE(B, true, R); else NF4K_MERGE(B, false, R);
  if (base == 0) {
    NF4K_MERGE_O(0, false)
  } else if (base == 1) {
    if (res) { NF4K_MERGE_O(1, true) } else { NF4K_MERGE_O(1, false) }
  } else {
    if (res) { NF4K_MERGE_O(2, true) } else { NF4K_MERGE_O(2, false) }
  }
#undef NF4K_MERGE_O
#undef NF4K_MERGE
  return hipGetLastError();
}

}  // namespace nf4k
