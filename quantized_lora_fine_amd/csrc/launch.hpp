// Kernel launchers of libnf4lora (implemented in the .hip files).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "nf4_host.hpp"

namespace nf4k {

enum { MODE_FWD = 0, MODE_DX = 1 };

// codes2/absmax2/dqs2: the residual (second-stage) tensor, or NULL for one stage.
hipError_t launch_quantize(const float* W, int64_t nblocks, bool dq, uint8_t* codes, void* absmax, float* dqs,
                           uint8_t* codes2, void* absmax2, float* dqs2, const NF4Enc& e, const NF4Consts& c,
                           hipStream_t st);
hipError_t launch_dequantize(const uint8_t* codes, const void* absmax, const float* dqs, const uint8_t* codes2,
                             const void* absmax2, const float* dqs2, int64_t nweights, bool dq, bool bf16, void* out,
                             const NF4Consts& c, hipStream_t st);
// nf4 quantize of one stage plus the reconstruction error of W (as launch_error
// computes it) from the same read of W; err_dq: error with the double-quantized
// scales (requires dq) rather than the plain block absmax.
hipError_t launch_quantize_error(const float* W, int64_t nblocks, bool dq, uint8_t* codes, void* absmax, float* dqs,
                                 bool err_dq, double* part, double* err, const NF4Enc& e, const NF4Consts& c,
                                 hipStream_t st);
hipError_t launch_error(const float* W, int64_t nblocks, bool dq, double* part, double* err, const NF4Enc& c,
                        hipStream_t st);
// launch_error for n linears (W[i], rows[i] x cols[i]) in batches of up to 64:
// err[i] as launch_error writes it for linear i, bit for bit; part holds one
// (D, Wn) pair per group of every linear, linear after linear.
hipError_t launch_error_batch(const float* const* W, const int64_t* rows, const int64_t* cols, int32_t n, bool dq,
                              double* part, double* err, const NF4Enc& c, hipStream_t st);
hipError_t launch_topk(const double* e, int n, int k, int* idx, hipStream_t st);
// Workspace of the allocation-free forward: one device array of this size per
// GPU (scratch.hip).  noalloc_scratch gives its address on the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void** ptr);

// MFMA-only probe: `workgroups` x 512 threads, each wave `iters` rounds of 8
// v_mfma_f32_32x32x16_bf16; out gets one float per thread.
hipError_t launch_mfma_peak(int iters, int workgroups, float* out, hipStream_t st);
// *flag_dev = 1 if any of W[0 .. count) is an infinity or a NaN, else 0.
hipError_t launch_check_finite(const float* W, int64_t count, int* flag_dev, hipStream_t st);

// The passes over W (quantize, error) run one 256-thread workgroup per group of
// 256 blocks; a launch holds at most kMaxLaunchGroups groups, so its work-item
// count (groups * 256) stays below 2^32.  Up to kErrBatch linears share one
// launch of the batched error pass.
constexpr int64_t kMaxLaunchGroups = ((int64_t)1 << 24) - 1;
constexpr int kErrBatch = 64;
inline int64_t error_groups(int64_t rows, int64_t cols) { return (rows * cols / 64 + 255) / 256; }
// The next launch of a batched error pass over n linears starts at linear c0
// and takes the k linears c0 .. c0 + k - 1 (the return value): as many as fit in
// kErrBatch linears and kMaxLaunchGroups groups.  g0[i] is the first group of
// linear c0 + i within the launch and g0[k] the launch's group count (g0 has
// kErrBatch + 1 entries).  Returns 0 when linear c0 alone has more than
// kMaxLaunchGroups groups.
int error_batch_chunk(const int64_t* rows, const int64_t* cols, int32_t n, int32_t c0, int64_t* g0);

// Weight source of the fused GEMM: NF4 with fp32 absmax, NF4 with 8-bit
// double-quantized scales, or a bf16 weight (no quantization).
enum { kSrcNF4 = 0, kSrcNF4DQ = 1, kSrcBF16 = 2 };
// Tail B2: [N][R] (b2kn == 0), or k-major [R][N] with rows b2kn .. R-1 absent (read as zero).
hipError_t launch_nf4_gemm(int mode, int src, const uint16_t* A, const uint16_t* Wb, const uint8_t* codes,
                           const void* absmax, const float* dqs, const uint8_t* codes2, const void* absmax2,
                           const float* dqs2, const uint16_t* A2, const uint16_t* B2, int R, int b2kn, uint16_t* C,
                           int64_t M, int N, int K, const NF4Consts& c, hipStream_t st);

// W' = base + s (L1 L2)^T into fp32 or bf16; base 0: fp32 W, 1: NF4, 2: NF4 with 8-bit scales.
hipError_t launch_merge(int base, const float* W, const uint8_t* codes, const void* absmax, const float* dqs,
                        const uint8_t* codes2, const void* absmax2, const float* dqs2, const uint16_t* L1,
                        const uint16_t* L2, int r, float s, int64_t rows, int64_t cols, bool out_bf16, void* out,
                        const NF4Consts& c, hipStream_t st);

// One launch of k_prep: up to kPrepPads layout copies and kPrepZeros clears.
// Unused jobs have orows * ocols == 0 / n == 0.
constexpr int kPrepPads = 3;
constexpr int kPrepZeros = 2;
struct PadJob {  // out[i][j] = (i < irows && j < jcols) ? in[i*si + j*sj] : 0, out is [orows][ocols]
  const uint16_t* in;
  uint16_t* out;
  int64_t si, sj, irows, jcols, orows, ocols;
};
struct ZeroJob {
  uint32_t* p;
  int64_t n;  // 32-bit words
};
struct PrepArgs {
  PadJob pad[kPrepPads];
  ZeroJob zero[kPrepZeros];
};
hipError_t launch_prep(const PrepArgs& a, hipStream_t st);

// NT skinny product with its split reduction: out = alpha * A[M][K] B[RP][K]^T.
struct NtArgs {
  const uint16_t* A;
  const uint16_t* B;
  int64_t M;
  int K;
  int ksplit, krange;
  float* part;      // [ksplit][M][RP] fp32 (unused if ksplit == 1)
  unsigned* cnt;    // [ceil(M/64)] zeroed counters
  int r;
  float alpha1;
  uint16_t* out1;   // [M][ld1], columns < r, or NULL
  int ld1;
  float alpha2;
  uint16_t* out2;   // [M][RP], or NULL
  int bkn;          // 0: B is [RP][K]; > 0: B is k-major [K][bkn] (its first r columns used;
                    // whole-K kernel only, bkn % 8 == 0)
};
// TN skinny product with its split reduction: out = alpha * P[M][:r]^T Q[M][N].
struct TnArgs {
  const uint16_t* P;  // [M][ldp], 16-byte aligned, ldp % 8 == 0, columns r .. ceil8(r)-1 zero
  int ldp, r;
  const uint16_t* Q;
  int64_t M;
  int N;
  int msplit;
  int64_t mrange;
  float* part;      // [msplit][RP][N] fp32 (unused if msplit == 1)
  unsigned* cnt;    // [ceil(N/64)] zeroed counters
  float alpha;
  int trans;        // 0: out [r][N]; 1: out [N][r]
  float* out;
};
void plan_nt(int64_t M, int K, int* ksplit, int* krange);
void plan_tn(int64_t M, int N, int* msplit, int64_t* mrange);
hipError_t launch_skinny_nt(const NtArgs& a, int RP, hipStream_t st);
hipError_t launch_skinny_tn(const TnArgs& a, int RP, hipStream_t st);
// two TN products over the same tokens in one launch when possible (b may be NULL)
hipError_t launch_skinny_tn2(const TnArgs& a, const TnArgs* b, int RP, hipStream_t st);
// true when the launchers above use the unsplit kernels (whole K / all tokens
// per workgroup), which need neither the partial buffers nor the counters
bool skinny_nt_whole(int64_t M, int RP);
bool skinny_tn_whole(int64_t M, int RP);
// the kernel one NT product takes (its contraction K; bkn: k-major B)
bool skinny_nt_use_whole(int64_t M, int K, int RP, bool bkn);
// column band of the all-token TN kernel for products of N0 and N1 columns
// (N1 = 0: one product): 64 (whole 128-byte lines of Q per load) when that
// still gives 192 workgroups or more, else 32
int skinny_tn_band(int N0, int N1);
// row panels per group of the fused GEMM's tile order for a contraction of K:
// 2 while 16 panels of 256 rows (the 8 XCDs' working set) stay within the
// Infinity Cache, i.e. K <= 16384, else 1
int gemm_group_m(int K);
// A launch holds at most 2^32 - 1 work-items.  Rows per launch of an NT
// product over M token rows: M itself up to kNtLaunchRows, else equal
// consecutive ranges, each a multiple of 64 rows and at least 2^22 rows (so
// that each range takes the kernel the full product would).
constexpr int64_t kNtLaunchRows = (int64_t)1 << 24;
int64_t nt_launch_rows(int64_t M);
// 256-row panels per launch of the fused GEMM with tiles_n column tiles
// (512 work-items per tile)
int64_t gemm_launch_panels(int64_t tiles_n);

}  // namespace nf4k
