// C ABI of libnf4lora: argument validation, workspace planning and the
// launch sequence of each entry point.  See include/nf4lora.h for the
// contract of every function.
#include "nf4lora.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "launch.hpp"

using namespace nf4k;

namespace {

constexpr int64_t kBlock = 64;
constexpr int64_t kGroup = 256;
constexpr size_t kCheckWorkspace = 256;  // nf4_check_finite: one int flag

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};
Range rng(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

int32_t round16(int32_t r) { return (r + 15) / 16 * 16; }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

nf4_status hip_status(hipError_t e) { return e == hipSuccess ? NF4_OK : NF4_ERR_HIP; }

#define NF4_TRY(expr)                    \
  do {                                   \
    hipError_t e_ = (expr);              \
    if (e_ != hipSuccess) return NF4_ERR_HIP; \
  } while (0)

// Sizes of the three buffers of a quantized tensor.
void tensor_sizes(int64_t rows, int64_t cols, int32_t dq, size_t* codes, size_t* absmax, size_t* dqs) {
  const int64_t n = rows * cols;
  const int64_t nb = n / kBlock;
  *codes = (size_t)(n / 2);
  if (dq == 0) {
    *absmax = (size_t)(4 * nb);
    *dqs = 0;
  } else {
    *absmax = (size_t)nb;
    *dqs = (size_t)(4 * ((nb + kGroup - 1) / kGroup));
  }
}

nf4_status check_shape(int64_t rows, int64_t cols, int32_t block, int32_t dq) {
  if (block != kBlock) return NF4_ERR_ARG;
  if (dq != 0 && dq != kGroup) return NF4_ERR_ARG;
  if (rows < 0 || cols < 0) return NF4_ERR_SHAPE;
  if (cols % kBlock != 0) return NF4_ERR_SHAPE;
  if (rows > 0 && cols > (((int64_t)1 << 40) / rows)) return NF4_ERR_SHAPE;
  return NF4_OK;
}

// The passes over an fp32 W launch one 256-thread workgroup per group of 256
// blocks: at most kMaxLaunchGroups groups keep a launch below 2^32 work-items.
nf4_status check_pass_weights(int64_t rows, int64_t cols) {
  return error_groups(rows, cols) > kMaxLaunchGroups ? NF4_ERR_SHAPE : NF4_OK;
}

nf4_status check_tensor(const nf4_tensor* q) {
  if (!q) return NF4_ERR_NULL;
  nf4_status st = check_shape(q->rows, q->cols, q->block, q->dq_group);
  if (st != NF4_OK) return st;
  if (q->codebook < 0 || q->codebook >= kCodebooks) return NF4_ERR_ARG;
  if (q->residual) {
    const nf4_tensor* r = q->residual;
    if (r->residual || r == q) return NF4_ERR_ARG;
    if (r->rows != q->rows || r->cols != q->cols || r->block != q->block || r->dq_group != q->dq_group ||
        r->codebook != q->codebook)
      return NF4_ERR_SHAPE;
    if (q->rows * q->cols > 0) {
      if (!r->codes || !r->absmax || (r->dq_group && !r->dq_scale)) return NF4_ERR_NULL;
      if (!aligned16(r->codes) || !aligned16(r->absmax) || (r->dq_group && !aligned16(r->dq_scale)))
        return NF4_ERR_ALIGN;
      size_t cb, ab, db;
      tensor_sizes(q->rows, q->cols, q->dq_group, &cb, &ab, &db);
      const Range a[3] = {rng(q->codes, cb), rng(q->absmax, ab), rng(q->dq_scale, db)};
      const Range b[3] = {rng(r->codes, cb), rng(r->absmax, ab), rng(r->dq_scale, db)};
      for (const Range& x : a)
        for (const Range& y : b)
          if (overlap(x, y)) return NF4_ERR_ALIAS;
    }
  }
  if (q->rows * q->cols > 0) {
    if (!q->codes || !q->absmax) return NF4_ERR_NULL;
    if (q->dq_group && !q->dq_scale) return NF4_ERR_NULL;
    if (!aligned16(q->codes) || !aligned16(q->absmax)) return NF4_ERR_ALIGN;
    if (q->dq_group && !aligned16(q->dq_scale)) return NF4_ERR_ALIGN;
  }
  return NF4_OK;
}

// ---------------------------------------------------------------------------
// workspace plans
// ---------------------------------------------------------------------------
struct FwdPlan {
  int32_t RP;
  int ks, kr;
  size_t off_l1t, off_l2t, off_ts, off_part, off_cnt, total;
  int64_t ncnt;  // 32-bit counters
};

FwdPlan plan_fwd(int64_t M, int64_t o, int64_t h, int32_t r) {
  FwdPlan p;
  p.RP = round16(r);
  plan_nt(M, (int)h, &p.ks, &p.kr);
  p.ncnt = (M + 63) / 64;
  size_t off = 0;
  p.off_l1t = off;
  off += align256((size_t)p.RP * h * 2);
  p.off_l2t = off;
  off += align256((size_t)o * p.RP * 2);
  p.off_ts = off;
  off += align256((size_t)M * p.RP * 2);
  p.off_part = off;
  off += align256((size_t)p.ks * M * p.RP * 4);
  p.off_cnt = off;
  off += align256((size_t)p.ncnt * 4);
  p.total = off;
  return p;
}

struct BwdPlan {
  int32_t RP;
  int ks_t, kr_t, ks_g, kr_g, ms2, ms1;
  int64_t mr2, mr1;
  size_t off_l1t, off_l1p, off_l2p, off_tb, off_g, off_pnt, off_p2, off_p1, off_cnt, total;
  // counters (32-bit) at off_cnt: T recompute [mb], G [mb], dL2 [o/64], dL1 [h/64]
  int64_t cnt_t, cnt_g, cnt_2, cnt_1, ncnt;
};

BwdPlan plan_bwd(int64_t M, int64_t o, int64_t h, int32_t r) {
  BwdPlan p;
  p.RP = round16(r);
  plan_nt(M, (int)h, &p.ks_t, &p.kr_t);
  plan_nt(M, (int)o, &p.ks_g, &p.kr_g);
  plan_tn(M, (int)o, &p.ms2, &p.mr2);
  plan_tn(M, (int)h, &p.ms1, &p.mr1);
  const int ksmax = p.ks_t > p.ks_g ? p.ks_t : p.ks_g;
  const int64_t mb = (M + 63) / 64;
  p.cnt_t = 0;
  p.cnt_g = mb;
  p.cnt_2 = 2 * mb;
  p.cnt_1 = 2 * mb + (o + 63) / 64;
  p.ncnt = p.cnt_1 + (h + 63) / 64;
  size_t off = 0;
  p.off_l1t = off;
  off += align256((size_t)p.RP * h * 2);
  p.off_l1p = off;
  off += align256((size_t)h * p.RP * 2);
  p.off_l2p = off;
  off += align256((size_t)p.RP * o * 2);
  p.off_tb = off;
  off += align256((size_t)M * p.RP * 2);
  p.off_g = off;
  off += align256((size_t)M * p.RP * 2);
  p.off_pnt = off;
  off += align256((size_t)ksmax * M * p.RP * 4);
  p.off_p2 = off;
  off += align256((size_t)p.ms2 * p.RP * o * 4);
  p.off_p1 = off;
  off += align256((size_t)p.ms1 * p.RP * h * 4);
  p.off_cnt = off;
  off += align256((size_t)p.ncnt * 4);
  p.total = off;
  return p;
}

PadJob pad_job(const uint16_t* in, int64_t si, int64_t sj, int64_t irows, int64_t jcols, uint16_t* out,
               int64_t orows, int64_t ocols) {
  PadJob j;
  j.in = in;
  j.out = out;
  j.si = si;
  j.sj = sj;
  j.irows = irows;
  j.jcols = jcols;
  j.orows = orows;
  j.ocols = ocols;
  return j;
}

size_t error_ws(int64_t rows, int64_t cols) {
  const int64_t nb = rows * cols / kBlock;
  const int64_t ng = (nb + kGroup - 1) / kGroup;
  return align256((size_t)(ng > 0 ? ng : 1) * 16);
}

// The frozen weight of a layer as the fused GEMM reads it: NF4 (with fp32 or
// double-quantized scales) or bf16.  rows = o, cols = h.
struct WSrc {
  int src;
  int codebook;
  int64_t rows, cols;
  const uint16_t* wb;
  const uint8_t* codes;
  const void* absmax;
  const float* dqs;
  const uint8_t* codes2;  // residual stage, or NULL
  const void* absmax2;
  const float* dqs2;
  Range buf[6];  // the weight's buffers, for the aliasing checks
};

// the buffers of a quantized tensor and of its residual stage (empty ranges when absent)
void tensor_ranges(const nf4_tensor* q, Range out[6]) {
  size_t cb, ab, db;
  tensor_sizes(q->rows, q->cols, q->dq_group, &cb, &ab, &db);
  out[0] = rng(q->codes, cb);
  out[1] = rng(q->absmax, ab);
  out[2] = rng(q->dq_scale, db);
  const nf4_tensor* r = q->residual;
  out[3] = rng(r ? r->codes : nullptr, r ? cb : 0);
  out[4] = rng(r ? r->absmax : nullptr, r ? ab : 0);
  out[5] = rng(r ? r->dq_scale : nullptr, r ? db : 0);
}

// The fused GEMM reads a 256-row tile of the activations (256 * K * 2 bytes)
// and, for the input gradient, all packed codes (rows * cols / 2 bytes)
// through 32-bit buffer ranges: both stay below 4 GiB with these limits.
constexpr int64_t kMaxLayerDim = (int64_t)1 << 22;
constexpr int64_t kMaxLayerWeights = (int64_t)1 << 32;
nf4_status layer_shape(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || rows % kBlock != 0 || cols % kBlock != 0) return NF4_ERR_SHAPE;
  if (rows > kMaxLayerDim || cols > kMaxLayerDim || rows * cols > kMaxLayerWeights) return NF4_ERR_SHAPE;
  return NF4_OK;
}

nf4_status wsrc_nf4(const nf4_tensor* W, WSrc* w) {
  nf4_status st = check_tensor(W);
  if (st != NF4_OK) return st;
  st = layer_shape(W->rows, W->cols);
  if (st != NF4_OK) return st;
  w->src = W->dq_group ? kSrcNF4DQ : kSrcNF4;
  w->codebook = W->codebook;
  w->rows = W->rows;
  w->cols = W->cols;
  w->wb = nullptr;
  w->codes = W->codes;
  w->absmax = W->absmax;
  w->dqs = W->dq_scale;
  w->codes2 = W->residual ? W->residual->codes : nullptr;
  w->absmax2 = W->residual ? W->residual->absmax : nullptr;
  w->dqs2 = W->residual ? W->residual->dq_scale : nullptr;
  tensor_ranges(W, w->buf);
  return NF4_OK;
}

nf4_status wsrc_bf16(const uint16_t* W, int64_t rows, int64_t cols, WSrc* w) {
  nf4_status st = layer_shape(rows, cols);
  if (st != NF4_OK) return st;
  if (rows * cols > (int64_t)INT32_MAX) return NF4_ERR_SHAPE;  // byte offsets stay below 4 GiB
  if (!W) return NF4_ERR_NULL;
  if (!aligned16(W)) return NF4_ERR_ALIGN;
  w->src = kSrcBF16;
  w->codebook = kCodebookNF4;
  w->rows = rows;
  w->cols = cols;
  w->wb = W;
  w->codes = nullptr;
  w->absmax = nullptr;
  w->dqs = nullptr;
  w->codes2 = nullptr;
  w->absmax2 = nullptr;
  w->dqs2 = nullptr;
  w->buf[0] = rng(W, (size_t)(rows * cols * 2));
  for (int i = 1; i < 6; ++i) w->buf[i] = rng(nullptr, 0);
  return NF4_OK;
}

nf4_status check_batch(int64_t M, int32_t r) {
  if (M < 0 || M > ((int64_t)1 << 31)) return NF4_ERR_SHAPE;
  if (r < 1 || r > 256) return NF4_ERR_SHAPE;
  return NF4_OK;
}

// B2 is [N][R], or k-major [R][N] with its first b2kn rows present (b2kn > 0)
hipError_t gemm(int mode, const WSrc& w, const uint16_t* A, const uint16_t* A2, const uint16_t* B2, int R,
                int b2kn, uint16_t* C, int64_t M, hipStream_t st) {
  const int64_t N = mode == MODE_FWD ? w.rows : w.cols;
  const int64_t K = mode == MODE_FWD ? w.cols : w.rows;
  return launch_nf4_gemm(mode, w.src, A, w.wb, w.codes, w.absmax, w.dqs, w.codes2, w.absmax2, w.dqs2, A2, B2, R,
                         b2kn, C, M, (int)N, (int)K, codebook_consts(w.codebook), st);
}

nf4_status layer_fwd(const WSrc& W, const uint16_t* X, int64_t M, const uint16_t* L1, const uint16_t* L2,
                            int32_t r, float s, uint16_t* Y, uint16_t* T_out, void* ws, size_t ws_bytes,
                            void* stream) {
  nf4_status st = check_batch(M, r);
  if (st != NF4_OK) return st;
  if (M == 0) return NF4_OK;
  if (!X || !L1 || !L2 || !Y) return NF4_ERR_NULL;
  if (!aligned16(X) || !aligned16(L1) || !aligned16(L2) || !aligned16(Y) || (T_out && !aligned16(T_out)))
    return NF4_ERR_ALIGN;
  const int64_t o = W.rows, h = W.cols;
  const FwdPlan p = plan_fwd(M, o, h, r);
  if (!ws) return NF4_ERR_WORKSPACE;
  if (ws_bytes < p.total) return NF4_ERR_WORKSPACE;
  if (!aligned16(ws)) return NF4_ERR_ALIGN;
  const Range ins[] = {rng(X, (size_t)M * h * 2), rng(L1, (size_t)h * r * 2), rng(L2, (size_t)r * o * 2),
                       W.buf[0], W.buf[1], W.buf[2], W.buf[3], W.buf[4], W.buf[5]};
  const Range outs[] = {rng(Y, (size_t)M * o * 2), rng(T_out, T_out ? (size_t)M * r * 2 : 0),
                        rng(ws, p.total)};
  for (const Range& a : outs) {
    for (const Range& b : ins)
      if (overlap(a, b)) return NF4_ERR_ALIAS;
  }
  if (overlap(outs[0], outs[1]) || overlap(outs[0], outs[2]) || overlap(outs[1], outs[2])) return NF4_ERR_ALIAS;

  hipStream_t hs = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  uint16_t* l1t = (uint16_t*)(w + p.off_l1t);
  uint16_t* l2t = (uint16_t*)(w + p.off_l2t);
  uint16_t* ts = (uint16_t*)(w + p.off_ts);
  float* part = (float*)(w + p.off_part);
  unsigned* cnt = (unsigned*)(w + p.off_cnt);
  if (skinny_nt_whole(M, p.RP) && r % 8 == 0) {
    // no prep launch: the whole-K product reads L1 as stored (k-major, staged and
    // read transposed in LDS) and the GEMM tail reads L2 as stored ([r][o])
    NtArgs nt{X, L1, M, (int)h, 1, (int)h, part, cnt, r, 1.0f, T_out, r, s, ts, r};
    NF4_TRY(launch_skinny_nt(nt, p.RP, hs));
    NF4_TRY(gemm(MODE_FWD, W, X, ts, L2, p.RP, r, Y, M, hs));
    return NF4_OK;
  }
  // one prep launch: L1^T [RP][h] (rows >= r zero), L2^T [o][RP] (columns >= r zero), counters
  PrepArgs pa{};
  pa.pad[0] = pad_job(L1, 1, r, r, h, l1t, p.RP, h);
  pa.pad[1] = pad_job(L2, 1, o, o, r, l2t, o, p.RP);
  if (!skinny_nt_use_whole(M, (int)h, p.RP, false)) pa.zero[0] = ZeroJob{cnt, p.ncnt};
  NF4_TRY(launch_prep(pa, hs));
  // T = X L1 (split K, fixed-order reduction) -> T_out (bf16) and s*T (bf16, padded)
  NtArgs nt{X, l1t, M, (int)h, p.ks, p.kr, part, cnt, r, 1.0f, T_out, r, s, ts};
  NF4_TRY(launch_skinny_nt(nt, p.RP, hs));
  // Y = X w_hat^T + (s T) L2
  NF4_TRY(gemm(MODE_FWD, W, X, ts, l2t, p.RP, 0, Y, M, hs));
  return NF4_OK;
}

nf4_status layer_bwd(const WSrc& W, const uint16_t* X, const uint16_t* dY, int64_t M, const uint16_t* L1,
                            const uint16_t* L2, int32_t r, float s, const uint16_t* T, uint16_t* dX, float* dL1,
                            float* dL2, void* ws, size_t ws_bytes, void* stream) {
  nf4_status st = check_batch(M, r);
  if (st != NF4_OK) return st;
  if (!dL1 || !dL2) return NF4_ERR_NULL;
  if (M > 0 && (!X || !dY || !L1 || !L2)) return NF4_ERR_NULL;
  const int64_t o = W.rows, h = W.cols;
  const BwdPlan p = plan_bwd(M, o, h, r);
  if (!ws) return NF4_ERR_WORKSPACE;
  if (ws_bytes < p.total) return NF4_ERR_WORKSPACE;
  if (!aligned16(ws) || !aligned16(dL1) || !aligned16(dL2)) return NF4_ERR_ALIGN;
  if (M > 0 && (!aligned16(X) || !aligned16(dY) || !aligned16(L1) || !aligned16(L2) || (T && !aligned16(T)) ||
                (dX && !aligned16(dX))))
    return NF4_ERR_ALIGN;
  const Range ins[] = {rng(X, (size_t)M * h * 2),     rng(dY, (size_t)M * o * 2),
                       rng(L1, (size_t)h * r * 2),    rng(L2, (size_t)r * o * 2),
                       rng(T, T ? (size_t)M * r * 2 : 0), W.buf[0],
                       W.buf[1],                      W.buf[2],
                       W.buf[3],                      W.buf[4], W.buf[5]};
  const Range outs[] = {rng(dX, dX ? (size_t)M * h * 2 : 0), rng(dL1, (size_t)h * r * 4),
                        rng(dL2, (size_t)r * o * 4), rng(ws, p.total)};
  for (const Range& a : outs) {
    for (const Range& b : ins)
      if (overlap(a, b)) return NF4_ERR_ALIAS;
  }
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return NF4_ERR_ALIAS;

  hipStream_t hs = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  unsigned* cnt = (unsigned*)(w + p.off_cnt);
  if (M == 0) {
    // empty token set: both adapter gradients are exactly zero
    PrepArgs pa{};
    pa.zero[0] = ZeroJob{(uint32_t*)dL2, (int64_t)r * o};
    pa.zero[1] = ZeroJob{(uint32_t*)dL1, (int64_t)h * r};
    NF4_TRY(launch_prep(pa, hs));
    return NF4_OK;
  }
  uint16_t* l1t = (uint16_t*)(w + p.off_l1t);
  uint16_t* l1p = (uint16_t*)(w + p.off_l1p);
  uint16_t* l2p = (uint16_t*)(w + p.off_l2p);
  uint16_t* tb = (uint16_t*)(w + p.off_tb);
  uint16_t* g = (uint16_t*)(w + p.off_g);
  float* pnt = (float*)(w + p.off_pnt);
  float* p2 = (float*)(w + p.off_p2);
  float* p1 = (float*)(w + p.off_p1);

  // one prep launch: L1 [h][RP] and L2 [RP][o] with zero padding (L1 and L2 are used
  // as they are when r is a multiple of 16), counters when a split product runs, and
  // L1^T [RP][h] when T is recomputed or T [M][RP] when the given T has rows that are
  // not whole 16-byte chunks
  PrepArgs pa{};
  const uint16_t* l1b = L1;
  const uint16_t* l2b = L2;
  if (r != p.RP) {
    pa.pad[0] = pad_job(L1, r, 1, h, r, l1p, h, p.RP);
    pa.pad[1] = pad_job(L2, o, 1, r, o, l2p, p.RP, o);
    l1b = l1p;
    l2b = l2p;
  }
  if (!T) pa.pad[2] = pad_job(L1, 1, r, r, h, l1t, p.RP, h);
  else if (r % 8 != 0) pa.pad[2] = pad_job(T, r, 1, M, r, tb, M, p.RP);
  if (!skinny_nt_use_whole(M, (int)h, p.RP, false) || !skinny_nt_use_whole(M, (int)o, p.RP, false) ||
      !skinny_tn_whole(M, p.RP))
    pa.zero[0] = ZeroJob{cnt, p.ncnt};
  NF4_TRY(launch_prep(pa, hs));
  const uint16_t* tsrc = T;
  int ldt = r;
  if (!T) {
    NtArgs nt{X, l1t, M, (int)h, p.ks_t, p.kr_t, pnt, cnt + p.cnt_t, r, 1.0f, nullptr, 0, 1.0f, tb};
    NF4_TRY(launch_skinny_nt(nt, p.RP, hs));
    tsrc = tb;
    ldt = p.RP;
  } else if (r % 8 != 0) {
    tsrc = tb;  // padded by the prep launch: the TN product reads rows in 16-byte chunks
    ldt = p.RP;
  }
  // G = s dY L2^T  (bf16 [M][RP], columns >= r zero)
  NtArgs ng{dY, l2b, M, (int)o, p.ks_g, p.kr_g, pnt, cnt + p.cnt_g, r, 1.0f, nullptr, 0, s, g};
  NF4_TRY(launch_skinny_nt(ng, p.RP, hs));
  // dL2 = s T^T dY  ([r][o]),  dL1 = X^T G  (stored [h][r])
  TnArgs t2{tsrc, ldt, r, dY, M, (int)o, p.ms2, p.mr2, p2, cnt + p.cnt_2, s, 0, dL2};
  TnArgs t1{g, p.RP, r, X, M, (int)h, p.ms1, p.mr1, p1, cnt + p.cnt_1, 1.0f, 1, dL1};
  // dX = dY w_hat + G L1^T, before the TN products: it reads dY right after G's
  // product has brought it into the caches, and the TN products then find dY there
  if (dX) {
    NF4_TRY(gemm(MODE_DX, W, dY, g, l1b, p.RP, 0, dX, M, hs));
  }
  NF4_TRY(launch_skinny_tn2(t2, &t1, p.RP, hs));
  return NF4_OK;
}

nf4_status wsrc_linear(const nf4_linear& L, WSrc* w) {
  if ((L.q != nullptr) == (L.w_bf16 != nullptr)) return NF4_ERR_ARG;  // exactly one weight
  return L.q ? wsrc_nf4(L.q, w) : wsrc_bf16(L.w_bf16, L.rows, L.cols, w);
}

// the base product alone (a linear without adapter): Y = X W^T, or dX = dY W
nf4_status plain_product(int mode, const WSrc& w, const uint16_t* A, uint16_t* C, int64_t M, void* stream) {
  if (M < 0 || M > ((int64_t)1 << 31)) return NF4_ERR_SHAPE;
  if (M == 0) return NF4_OK;
  if (!A || !C) return NF4_ERR_NULL;
  if (!aligned16(A) || !aligned16(C)) return NF4_ERR_ALIGN;
  const int64_t K = mode == MODE_FWD ? w.cols : w.rows, N = mode == MODE_FWD ? w.rows : w.cols;
  const Range out = rng(C, (size_t)M * N * 2);
  if (overlap(out, rng(A, (size_t)M * K * 2))) return NF4_ERR_ALIAS;
  for (const Range& b : w.buf)
    if (overlap(out, b)) return NF4_ERR_ALIAS;
  return hip_status(gemm(mode, w, A, nullptr, nullptr, 0, 0, C, M, (hipStream_t)stream));
}

// Shapes of a batched error pass: every linear as nf4_layer_error checks it,
// and the partial slots of all of them (16 bytes each) in *need.
nf4_status error_batch_shapes(const int64_t* rows, const int64_t* cols, int32_t n, size_t* need) {
  if (n < 0) return NF4_ERR_ARG;
  if (n > 0 && (!rows || !cols)) return NF4_ERR_NULL;
  int64_t slots = 0;
  for (int32_t i = 0; i < n; ++i) {
    nf4_status st = check_shape(rows[i], cols[i], kBlock, 0);
    if (st == NF4_OK) st = check_pass_weights(rows[i], cols[i]);
    if (st != NF4_OK) return st;
    slots += (rows[i] * cols[i] / kBlock + kGroup - 1) / kGroup;
  }
  *need = align256((size_t)(slots > 0 ? slots : 1) * 16);
  return NF4_OK;
}

}  // namespace

extern "C" {

int nf4_abi_version(void) { return NF4LORA_ABI_VERSION; }

const char* nf4_status_str(int s) {
  switch (s) {
    case NF4_OK: return "NF4_OK";
    case NF4_ERR_NULL: return "NF4_ERR_NULL: a required pointer is NULL";
    case NF4_ERR_SHAPE: return "NF4_ERR_SHAPE: a size is out of range or the sizes disagree";
    case NF4_ERR_ALIGN: return "NF4_ERR_ALIGN: a device pointer is not 16-byte aligned";
    case NF4_ERR_WORKSPACE: return "NF4_ERR_WORKSPACE: workspace missing or too small";
    case NF4_ERR_ALIAS: return "NF4_ERR_ALIAS: an output overlaps an input";
    case NF4_ERR_HIP: return "NF4_ERR_HIP: a HIP call or kernel launch failed";
    case NF4_ERR_ARG: return "NF4_ERR_ARG: unsupported option";
    case NF4_ERR_NONFINITE: return "NF4_ERR_NONFINITE: the weight holds an infinity or a NaN";
    default: return "unknown nf4_status";
  }
}

nf4_status nf4_codebook_values(int32_t codebook, float out[16]) {
  if (!out) return NF4_ERR_NULL;
  if (codebook < 0 || codebook >= kCodebooks) return NF4_ERR_ARG;
  std::memcpy(out, codebook_consts(codebook).table, sizeof(float) * 16);
  return NF4_OK;
}

void nf4_code_table(float out[16]) {
  if (!out) return;
  const NF4Consts& c = nf4_consts();
  std::memcpy(out, c.table, sizeof(c.table));
}

nf4_status nf4_tensor_bytes(int64_t rows, int64_t cols, int32_t block, int32_t dq_group, size_t* codes_bytes,
                            size_t* absmax_bytes, size_t* dq_scale_bytes) {
  nf4_status st = check_shape(rows, cols, block, dq_group);
  if (st != NF4_OK) return st;
  size_t c, a, d;
  tensor_sizes(rows, cols, dq_group, &c, &a, &d);
  if (codes_bytes) *codes_bytes = c;
  if (absmax_bytes) *absmax_bytes = a;
  if (dq_scale_bytes) *dq_scale_bytes = d;
  return NF4_OK;
}

nf4_status nf4_quantize(const float* W, const nf4_tensor* q, void* stream) {
  nf4_status st = check_tensor(q);
  if (st != NF4_OK) return st;
  st = check_pass_weights(q->rows, q->cols);
  if (st != NF4_OK) return st;
  const int64_t n = q->rows * q->cols;
  if (n == 0) return NF4_OK;
  if (!W) return NF4_ERR_NULL;
  if (!aligned16(W)) return NF4_ERR_ALIGN;
  Range bufs[6];
  tensor_ranges(q, bufs);
  const Range in = rng(W, (size_t)n * 4);
  for (int i = 0; i < 6; ++i) {
    if (overlap(in, bufs[i])) return NF4_ERR_ALIAS;
    for (int j = i + 1; j < 6; ++j)
      if (overlap(bufs[i], bufs[j])) return NF4_ERR_ALIAS;
  }
  const nf4_tensor* r = q->residual;
  return hip_status(launch_quantize(W, n / kBlock, q->dq_group != 0, q->codes, q->absmax, q->dq_scale,
                                    r ? r->codes : nullptr, r ? r->absmax : nullptr, r ? r->dq_scale : nullptr,
                                    codebook_enc(q->codebook), codebook_consts(q->codebook), (hipStream_t)stream));
}

nf4_status nf4_dequantize(const nf4_tensor* q, void* W_out, int32_t out_is_bf16, void* stream) {
  nf4_status st = check_tensor(q);
  if (st != NF4_OK) return st;
  const int64_t n = q->rows * q->cols;
  if (n == 0) return NF4_OK;
  if (!W_out) return NF4_ERR_NULL;
  if (!aligned16(W_out)) return NF4_ERR_ALIGN;
  Range bufs[6];
  tensor_ranges(q, bufs);
  const Range out = rng(W_out, (size_t)n * (out_is_bf16 ? 2 : 4));
  for (const Range& b : bufs)
    if (overlap(out, b)) return NF4_ERR_ALIAS;
  const nf4_tensor* r = q->residual;
  return hip_status(launch_dequantize(q->codes, q->absmax, q->dq_scale, r ? r->codes : nullptr,
                                      r ? r->absmax : nullptr, r ? r->dq_scale : nullptr, n, q->dq_group != 0,
                                      out_is_bf16 != 0, W_out, codebook_consts(q->codebook), (hipStream_t)stream));
}

nf4_status nf4_workspace_bytes(int32_t op, int64_t M, int64_t rows, int64_t cols, int32_t r, size_t* bytes) {
  if (!bytes) return NF4_ERR_NULL;
  if (op == NF4_OP_CHECK) {
    *bytes = kCheckWorkspace;
    return NF4_OK;
  }
  if (op == NF4_OP_ERROR) {
    nf4_status st = check_shape(rows, cols, kBlock, 0);
    if (st != NF4_OK) return st;
    *bytes = error_ws(rows, cols);
    return NF4_OK;
  }
  if (op != NF4_OP_FWD && op != NF4_OP_BWD) return NF4_ERR_ARG;
  if (rows <= 0 || cols <= 0 || rows % kBlock || cols % kBlock || M < 0 || r < 1 || r > 256) return NF4_ERR_SHAPE;
  *bytes = (op == NF4_OP_FWD) ? plan_fwd(M, rows, cols, r).total : plan_bwd(M, rows, cols, r).total;
  return NF4_OK;
}

nf4_status nf4lora_fwd(const nf4_tensor* W, const uint16_t* X, int64_t M, const uint16_t* L1, const uint16_t* L2,
                       int32_t r, float s, uint16_t* Y, uint16_t* T_out, void* ws, size_t ws_bytes, void* stream) {
  WSrc w;
  nf4_status st = wsrc_nf4(W, &w);
  if (st != NF4_OK) return st;
  return layer_fwd(w, X, M, L1, L2, r, s, Y, T_out, ws, ws_bytes, stream);
}

nf4_status nf4lora_fwd_noalloc(const nf4_tensor* W, const uint16_t* X, int64_t M, const uint16_t* L1,
                               const uint16_t* L2, int32_t r, float s, uint16_t* Y, uint16_t* T_out, void* stream) {
  WSrc w;
  nf4_status st = wsrc_nf4(W, &w);
  if (st != NF4_OK) return st;
  st = check_batch(M, r);
  if (st != NF4_OK) return st;
  if (M == 0) return NF4_OK;
  // the plan must fit the fixed area; checked before any HIP call
  if (plan_fwd(M, w.rows, w.cols, r).total > kNoAllocScratchBytes) return NF4_ERR_WORKSPACE;
  void* ws = nullptr;
  NF4_TRY(noalloc_scratch(&ws));
  return layer_fwd(w, X, M, L1, L2, r, s, Y, T_out, ws, kNoAllocScratchBytes, stream);
}

nf4_status nf4lora_bwd(const nf4_tensor* W, const uint16_t* X, const uint16_t* dY, int64_t M, const uint16_t* L1,
                       const uint16_t* L2, int32_t r, float s, const uint16_t* T, uint16_t* dX, float* dL1,
                       float* dL2, void* ws, size_t ws_bytes, void* stream) {
  WSrc w;
  nf4_status st = wsrc_nf4(W, &w);
  if (st != NF4_OK) return st;
  return layer_bwd(w, X, dY, M, L1, L2, r, s, T, dX, dL1, dL2, ws, ws_bytes, stream);
}

nf4_status bf16lora_fwd(const uint16_t* W, int64_t rows, int64_t cols, const uint16_t* X, int64_t M,
                        const uint16_t* L1, const uint16_t* L2, int32_t r, float s, uint16_t* Y, uint16_t* T_out,
                        void* ws, size_t ws_bytes, void* stream) {
  WSrc w;
  nf4_status st = wsrc_bf16(W, rows, cols, &w);
  if (st != NF4_OK) return st;
  return layer_fwd(w, X, M, L1, L2, r, s, Y, T_out, ws, ws_bytes, stream);
}

nf4_status bf16lora_bwd(const uint16_t* W, int64_t rows, int64_t cols, const uint16_t* X, const uint16_t* dY,
                        int64_t M, const uint16_t* L1, const uint16_t* L2, int32_t r, float s, const uint16_t* T,
                        uint16_t* dX, float* dL1, float* dL2, void* ws, size_t ws_bytes, void* stream) {
  WSrc w;
  nf4_status st = wsrc_bf16(W, rows, cols, &w);
  if (st != NF4_OK) return st;
  return layer_bwd(w, X, dY, M, L1, L2, r, s, T, dX, dL1, dL2, ws, ws_bytes, stream);
}

nf4_status nf4_matmul(const nf4_tensor* W, int32_t transpose, const uint16_t* A, int64_t M, const uint16_t* A2,
                      const uint16_t* B2, int32_t R, uint16_t* C, void* stream) {
  nf4_status st = check_tensor(W);
  if (st != NF4_OK) return st;
  st = layer_shape(W->rows, W->cols);
  if (st != NF4_OK) return st;
  if (transpose != 0 && transpose != 1) return NF4_ERR_ARG;
  if (M < 0 || M > ((int64_t)1 << 31) || R < 0 || R > 256 || R % 16 != 0) return NF4_ERR_SHAPE;
  if (M == 0) return NF4_OK;
  if (!A || !C || (R > 0 && (!A2 || !B2))) return NF4_ERR_NULL;
  if (!aligned16(A) || !aligned16(C) || (R > 0 && (!aligned16(A2) || !aligned16(B2)))) return NF4_ERR_ALIGN;
  const int64_t o = W->rows, h = W->cols;
  const int64_t K = transpose ? o : h, N = transpose ? h : o;
  WSrc w;
  st = wsrc_nf4(W, &w);
  if (st != NF4_OK) return st;
  const Range out = rng(C, (size_t)M * N * 2);
  const Range ins[] = {rng(A, (size_t)M * K * 2), rng(A2, R ? (size_t)M * R * 2 : 0), rng(B2, R ? (size_t)N * R * 2 : 0)};
  for (const Range& b : ins)
    if (overlap(out, b)) return NF4_ERR_ALIAS;
  for (const Range& b : w.buf)
    if (overlap(out, b)) return NF4_ERR_ALIAS;
  return hip_status(gemm(transpose ? MODE_DX : MODE_FWD, w, A, A2, B2, R, 0, C, M, (hipStream_t)stream));
}

nf4_status nf4_layer_error(const float* W, int64_t rows, int64_t cols, int32_t block, int32_t dq_group,
                           int32_t codebook, double* err_dev, void* ws, size_t ws_bytes, void* stream) {
  nf4_status st = check_shape(rows, cols, block, dq_group);
  if (st != NF4_OK) return st;
  st = check_pass_weights(rows, cols);
  if (st != NF4_OK) return st;
  if (codebook < 0 || codebook >= kCodebooks) return NF4_ERR_ARG;
  if (!err_dev) return NF4_ERR_NULL;
  const int64_t n = rows * cols;
  if (n > 0 && !W) return NF4_ERR_NULL;
  if (!ws) return NF4_ERR_WORKSPACE;
  const size_t need = error_ws(rows, cols);
  if (ws_bytes < need) return NF4_ERR_WORKSPACE;
  if ((W && !aligned16(W)) || !aligned16(ws) || !aligned16(err_dev)) return NF4_ERR_ALIGN;
  const Range in = rng(W, (size_t)n * 4);
  if (overlap(in, rng(ws, need)) || overlap(in, rng(err_dev, 8)) || overlap(rng(ws, need), rng(err_dev, 8)))
    return NF4_ERR_ALIAS;
  return hip_status(launch_error(W, n / kBlock, dq_group != 0, (double*)ws, err_dev, codebook_enc(codebook),
                                 (hipStream_t)stream));
}

nf4_status nf4_error_batch_workspace_bytes(const int64_t* rows, const int64_t* cols, int32_t n, size_t* bytes) {
  if (!bytes) return NF4_ERR_NULL;
  return error_batch_shapes(rows, cols, n, bytes);
}

nf4_status nf4_layer_error_batch(const float* const* W, const int64_t* rows, const int64_t* cols, int32_t n,
                                 int32_t dq_group, int32_t codebook, double* err_dev, void* ws, size_t ws_bytes,
                                 void* stream) {
  size_t need = 0;
  nf4_status st = error_batch_shapes(rows, cols, n, &need);
  if (st != NF4_OK) return st;
  if (dq_group != 0 && dq_group != kGroup) return NF4_ERR_ARG;
  if (codebook < 0 || codebook >= kCodebooks) return NF4_ERR_ARG;
  if (n == 0) return NF4_OK;
  if (!W || !err_dev) return NF4_ERR_NULL;
  if (!ws) return NF4_ERR_WORKSPACE;
  if (ws_bytes < need) return NF4_ERR_WORKSPACE;
  if (!aligned16(ws) || ((uintptr_t)err_dev & 7u) != 0) return NF4_ERR_ALIGN;
  const Range wr = rng(ws, need), er = rng(err_dev, (size_t)n * 8);
  if (overlap(wr, er)) return NF4_ERR_ALIAS;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t cnt = rows[i] * cols[i];
    if (cnt > 0 && !W[i]) return NF4_ERR_NULL;
    if (W[i] && !aligned16(W[i])) return NF4_ERR_ALIGN;
    const Range in = rng(W[i], (size_t)cnt * 4);
    if (overlap(in, wr) || overlap(in, er)) return NF4_ERR_ALIAS;
  }
  return hip_status(launch_error_batch(W, rows, cols, n, dq_group != 0, (double*)ws, err_dev,
                                       codebook_enc(codebook), (hipStream_t)stream));
}

nf4_status nf4_quantize_error(const float* W, const nf4_tensor* q, int32_t err_dq_group, double* err_dev, void* ws,
                              size_t ws_bytes, void* stream) {
  nf4_status st = check_tensor(q);
  if (st != NF4_OK) return st;
  st = check_pass_weights(q->rows, q->cols);
  if (st != NF4_OK) return st;
  if (q->residual) return NF4_ERR_ARG;
  if (err_dq_group != 0 && err_dq_group != q->dq_group) return NF4_ERR_ARG;
  if (!err_dev) return NF4_ERR_NULL;
  const int64_t n = q->rows * q->cols;
  if (n > 0 && !W) return NF4_ERR_NULL;
  if (!ws) return NF4_ERR_WORKSPACE;
  const size_t need = error_ws(q->rows, q->cols);
  if (ws_bytes < need) return NF4_ERR_WORKSPACE;
  if ((W && !aligned16(W)) || !aligned16(ws) || !aligned16(err_dev)) return NF4_ERR_ALIGN;
  Range bufs[8];
  tensor_ranges(q, bufs);
  bufs[6] = rng(ws, need);
  bufs[7] = rng(err_dev, 8);
  const Range in = rng(W, (size_t)n * 4);
  for (int i = 0; i < 8; ++i) {
    if (overlap(in, bufs[i])) return NF4_ERR_ALIAS;
    for (int j = i + 1; j < 8; ++j)
      if (overlap(bufs[i], bufs[j])) return NF4_ERR_ALIAS;
  }
  return hip_status(launch_quantize_error(W, n / kBlock, q->dq_group != 0, q->codes, q->absmax, q->dq_scale,
                                          err_dq_group != 0, (double*)ws, err_dev, codebook_enc(q->codebook),
                                          codebook_consts(q->codebook), (hipStream_t)stream));
}

nf4_status nf4_check_finite(const float* W, int64_t count, void* ws, size_t ws_bytes, void* stream) {
  if (count < 0) return NF4_ERR_SHAPE;
  if (count == 0) return NF4_OK;
  if (!W) return NF4_ERR_NULL;
  if (!ws || ws_bytes < kCheckWorkspace) return NF4_ERR_WORKSPACE;
  if (!aligned16(W) || !aligned16(ws)) return NF4_ERR_ALIGN;
  if (overlap(rng(W, (size_t)count * 4), rng(ws, kCheckWorkspace))) return NF4_ERR_ALIAS;
  hipStream_t hs = (hipStream_t)stream;
  int* flag = (int*)ws;
  NF4_TRY(launch_check_finite(W, count, flag, hs));
  int host = 0;
  NF4_TRY(hipMemcpyAsync(&host, flag, sizeof(int), hipMemcpyDeviceToHost, hs));
  NF4_TRY(hipStreamSynchronize(hs));
  return host ? NF4_ERR_NONFINITE : NF4_OK;
}

nf4_status nf4_topk(const double* err_dev, int32_t n, int32_t k, int32_t* idx_dev, void* stream) {
  if (n < 0 || k < 0 || k > n || n > 65536) return NF4_ERR_SHAPE;
  if (k == 0) return NF4_OK;
  if (!err_dev || !idx_dev) return NF4_ERR_NULL;
  if (!aligned16(err_dev) || !aligned16(idx_dev)) return NF4_ERR_ALIGN;
  if (overlap(rng(err_dev, (size_t)n * 8), rng(idx_dev, (size_t)k * 4))) return NF4_ERR_ALIAS;
  return hip_status(launch_topk(err_dev, n, k, idx_dev, (hipStream_t)stream));
}

nf4_status nf4_probe_mfma_peak(int32_t iters, int32_t workgroups, float* out_dev, void* stream) {
  if (iters < 1 || workgroups < 1 || workgroups > (1 << 20)) return NF4_ERR_SHAPE;
  if (!out_dev) return NF4_ERR_NULL;
  if (!aligned16(out_dev)) return NF4_ERR_ALIGN;
  return hip_status(launch_mfma_peak(iters, workgroups, out_dev, (hipStream_t)stream));
}

int32_t nf4_protect_count(double rho, int32_t n) {
  if (!(rho >= 0.0 && rho <= 1.0) || n < 0) return -1;
  return (int32_t)std::floor(rho * (double)n + 0.5);
}


nf4_status nf4_stack_workspace_bytes(const nf4_linear* layers, int32_t n, int64_t M, size_t* bytes) {
  if (!bytes || (n > 0 && !layers)) return NF4_ERR_NULL;
  if (n < 0 || M < 0) return NF4_ERR_SHAPE;
  size_t most = 0;
  for (int32_t i = 0; i < n; ++i) {
    const nf4_linear& L = layers[i];
    WSrc w;
    nf4_status st = wsrc_linear(L, &w);
    if (st != NF4_OK) return st;
    if (L.r == 0) continue;
    if (L.r < 0 || L.r > 256) return NF4_ERR_SHAPE;
    const size_t f = plan_fwd(M, w.rows, w.cols, L.r).total, b = plan_bwd(M, w.rows, w.cols, L.r).total;
    most = std::max(most, std::max(f, b));
  }
  *bytes = most;
  return NF4_OK;
}

nf4_status nf4_stack_fwd(const nf4_linear* layers, int32_t n, int64_t M, void* ws, size_t ws_bytes, void* stream) {
  if (n > 0 && !layers) return NF4_ERR_NULL;
  if (n < 0) return NF4_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    const nf4_linear& L = layers[i];
    WSrc w;
    nf4_status st = wsrc_linear(L, &w);
    if (st == NF4_OK) {
      st = L.r == 0 ? plain_product(MODE_FWD, w, L.X, L.Y, M, stream)
                    : layer_fwd(w, L.X, M, L.L1, L.L2, L.r, L.s, L.Y, L.T, ws, ws_bytes, stream);
    }
    if (st != NF4_OK) return st;
  }
  return NF4_OK;
}

nf4_status nf4_stack_bwd(const nf4_linear* layers, int32_t n, int32_t cut, int64_t M, void* ws, size_t ws_bytes,
                         void* stream) {
  if (n > 0 && !layers) return NF4_ERR_NULL;
  if (n < 0 || cut < 0 || cut > n) return NF4_ERR_SHAPE;
  for (int32_t i = n - 1; i >= cut; --i) {
    const nf4_linear& L = layers[i];
    WSrc w;
    nf4_status st = wsrc_linear(L, &w);
    if (st == NF4_OK) {
      if (L.r == 0) {
        if (L.dX) st = plain_product(MODE_DX, w, L.dY, L.dX, M, stream);
      } else {
        st = layer_bwd(w, L.X, L.dY, M, L.L1, L.L2, L.r, L.s, L.T, L.dX, L.dL1, L.dL2, ws, ws_bytes, stream);
      }
    }
    if (st != NF4_OK) return st;
  }
  return NF4_OK;
}


nf4_status nf4lora_merge(const float* W, const nf4_tensor* q, int64_t rows, int64_t cols, const uint16_t* L1,
                         const uint16_t* L2, int32_t r, float s, void* W_out, int32_t out_is_bf16, void* stream) {
  nf4_status st = check_shape(rows, cols, (int32_t)kBlock, 0);
  if (st != NF4_OK) return st;
  if (r < 1 || r > 256) return NF4_ERR_SHAPE;
  if (rows > INT32_MAX / 2 || cols > INT32_MAX / 2) return NF4_ERR_SHAPE;
  const int64_t n = rows * cols;
  Range wb[6];
  for (Range& x : wb) x = rng(nullptr, 0);
  int base = 0;
  if (!W) {
    if (!q) return NF4_ERR_NULL;
    st = check_tensor(q);
    if (st != NF4_OK) return st;
    if (q->rows != rows || q->cols != cols) return NF4_ERR_SHAPE;
    tensor_ranges(q, wb);
    base = q->dq_group ? 2 : 1;
  } else {
    if (!aligned16(W)) return NF4_ERR_ALIGN;
    wb[0] = rng(W, (size_t)n * 4);
  }
  if (n == 0) return NF4_OK;
  if (!L1 || !L2 || !W_out) return NF4_ERR_NULL;
  if (!aligned16(W_out) || !aligned16(L1) || !aligned16(L2)) return NF4_ERR_ALIGN;
  const Range out = rng(W_out, (size_t)n * (out_is_bf16 ? 2 : 4));
  if (overlap(out, rng(L1, (size_t)cols * r * 2)) || overlap(out, rng(L2, (size_t)r * rows * 2)))
    return NF4_ERR_ALIAS;
  for (const Range& b : wb)
    if (overlap(out, b)) return NF4_ERR_ALIAS;
  const nf4_tensor* qq = W ? nullptr : q;  // the NF4 base, when the fp32 base is absent
  const nf4_tensor* rr = qq ? qq->residual : nullptr;
  return hip_status(launch_merge(base, W, qq ? qq->codes : nullptr, qq ? qq->absmax : nullptr,
                                 qq ? qq->dq_scale : nullptr, rr ? rr->codes : nullptr, rr ? rr->absmax : nullptr,
                                 rr ? rr->dq_scale : nullptr, L1, L2, r, s, rows, cols, out_is_bf16 != 0, W_out,
                                 codebook_consts(qq ? qq->codebook : 0), (hipStream_t)stream));
}

}  // extern "C"
