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

hipError_t launch_merge(int base, const float* W, const uint8_t* codes, const void* absmax, const float* dqs,
                        const uint8_t* codes2, const void* absmax2, const float* dqs2, const uint16_t* L1,
                        const uint16_t* L2, int r, float s, int64_t rows, int64_t cols, bool out_bf16, void* out,
                        const NF4Consts& c, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const dim3 gr((unsigned)((cols + MG_COLS - 1) / MG_COLS), (unsigned)((rows + MG_ROWS - 1) / MG_ROWS)), bl(256);
  const bool res = base != 0 && codes2 != nullptr;
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
