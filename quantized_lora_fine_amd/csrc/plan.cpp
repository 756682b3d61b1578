// Launch planning of libnf4lora: how the skinny adapter products split their
// contraction, and how the batched error pass groups linears into launches.
// Host code only (no kernels), so the C ABI layer and its CPU-only tests
// link it without a GPU.
#include "launch.hpp"

namespace nf4k {

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


// whole-K workgroups when the rank is small and there are rows enough for them
bool skinny_nt_whole(int64_t M, int RP) {
  if (RP > 64) return false;
  const int rw = RP <= 16 ? 8 : (RP <= 32 ? 16 : 32);
  return (M + rw - 1) / rw >= 64;
}

// The whole-K kernel for one NT product, given its contraction K and B layout.
// A k-major B takes it always.  A rank-64 product with a long contraction over
// many rows (G at 8192+ tokens against 8192+ outputs) takes the split kernel
// instead: a whole-K workgroup of 32 rows reads the entire 64 x K operand from
// L2, a split workgroup of 64 rows half of that per row.
bool skinny_nt_use_whole(int64_t M, int K, int RP, bool bkn) {
  if (!skinny_nt_whole(M, RP)) return false;
  if (bkn) return true;
  return !(RP == 64 && M >= 8192 && K >= 8192);
}

// all tokens per workgroup when the rank is small and the token count is not tiny
bool skinny_tn_whole(int64_t M, int RP) { return RP <= 64 && M >= 512; }

int skinny_tn_band(int N0, int N1) {
  const int64_t wide = ((int64_t)N0 + 63) / 64 + ((int64_t)N1 + 63) / 64;
  return wide >= 192 ? 64 : 32;
}

int gemm_group_m(int K) { return K <= 16384 ? 2 : 1; }

int64_t nt_launch_rows(int64_t M) {
  if (M <= kNtLaunchRows) return M;
  const int64_t n = (M + kNtLaunchRows - 1) / kNtLaunchRows;
  return ((M + n - 1) / n + 63) / 64 * 64;
}

int64_t gemm_launch_panels(int64_t tiles_n) {
  const int64_t per = ((int64_t)0xFFFFFFFF / 512) / (tiles_n > 0 ? tiles_n : 1);
  return per > 0 ? per : 1;
}


int error_batch_chunk(const int64_t* rows, const int64_t* cols, int32_t n, int32_t c0, int64_t* g0) {
  int k = 0;
  g0[0] = 0;
  while (k < kErrBatch && c0 + k < n) {
    const int64_t end = g0[k] + error_groups(rows[c0 + k], cols[c0 + k]);
    if (end > kMaxLaunchGroups) break;
    g0[k + 1] = end;
    ++k;
  }
  return k;
}

}  // namespace nf4k
