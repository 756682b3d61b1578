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
//
// Why no release/acquire pair.  In the C++/HIP memory model the partials
// would be published by a release on the counter increment and read after an
// acquire by the last arrival.  At agent scope on this chip a release is a
// write-back of the whole L2 of the issuing XCD and an acquire an invalidate
// of it, per workgroup: that made these kernels about 5x slower.  The
// exchange instead relies on three properties of the hardware, each kept in
// this function and its two helpers:
//   1. every partial is written and read only with agent-scope atomic stores
//      and loads (st_/ld_shared_partial), which are coherent across XCDs: the
//      stores write through the XCD's L2 and the loads do not hit a stale L2
//      line;
//   2. s_waitcnt vmcnt(0) before the barrier waits for the acknowledgement of
//      each thread's stores, which arrives only once the store is visible at
//      the agent coherence point, so every partial of the workgroup is visible
//      before thread 0 issues the increment (the signal fence keeps the
//      compiler from moving the stores past it);
//   3. the increment is an agent-scope atomic on one counter; the workgroup
//      that reads nsplit - 1 is ordered after every other increment, hence
//      after every other workgroup's partials, and its partial loads are
//      issued only after the increment returned (they depend on s_last
//      through the barrier and the branch).
// A change of architecture or of the scopes above needs this argument
// redone; with a true release/acquire the code would stay correct at the
// cost above.
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
        if (kv && aval[a]) v = *(const u32x4*)(arow[a] + k + kq);
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
// NT skinny, whole K per workgroup (RP <= 64): the same product as k_skinny_nt
// without a split: a 1024-thread workgroup owns RW rows of A (RW = 8, 16 or 32,
// so that the B bytes it reads from L2 are at most twice its A bytes) and all
// of K.  Its 16 waves take interleaved K steps of 32 (at each unrolled step the
// workgroup streams 512 contiguous columns of its rows), U steps per round
// with every load of the round in flight, so a few hundred workgroups keep
// enough bytes in flight to stream A at HBM speed.  The 16 wave tiles are
// added in LDS in wave order; no partials, counters or second pass.
// With RW = 8 the MFMA A operand's rows 8..15 are zero.
// ---------------------------------------------------------------------------
template <int RPT>
struct NtRows {
  static constexpr int RW = RPT <= 16 ? 8 : (RPT <= 32 ? 16 : 32);
  static constexpr int FRA = RW >= 16 ? RW / 16 : 1;    // A fragments of 16 rows
  static constexpr int NJ = RPT / 16;
  static constexpr int U = 16 / (FRA + NJ);             // K steps per wave per round
  // k-major B: each wave stages one K step of B (32 rows x RPT) in LDS, rows
  // padded so a transposing read's 4 rows fall on distinct banks
  static constexpr int ROWB = RPT * 2 + (RPT * 2 % 128 == 0 ? 16 : 0);
  static constexpr int PPR = RPT / 8;                   // 16-byte pieces per B row
  static constexpr int BL = (32 * PPR + 63) / 64;       // B loads per lane per K step
  static constexpr int RED = 16 * RW * RPT * 4, STG = 16 * 32 * ROWB;
  static constexpr int SMEM = RED > STG ? RED : STG;
};

template <int RPT, bool BKN>
__global__ __launch_bounds__(1024) void k_skinny_nt_rows(NtArgs p) {
  using S = NtRows<RPT>;
  constexpr int RW = S::RW, FRA = S::FRA, NJ = S::NJ, U = S::U;
  constexpr int ROWB = S::ROWB, PPR = S::PPR, BL = S::BL;
  __shared__ __attribute__((aligned(16))) uint8_t smem[BKN ? S::SMEM : S::RED];
  float* red = (float*)smem;
  uint8_t* stage = smem + (BKN ? (threadIdx.x >> 6) * 32 * ROWB : 0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * RW;
  const int64_t M = p.M;
  const int K = p.K;
  const int li = lane & 15;
  const int kq = (lane >> 4) * 8;

  floatx4 acc[FRA][NJ];
#pragma unroll
  for (int a = 0; a < FRA; ++a)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[a][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* arow[FRA];
  bool aval[FRA];
#pragma unroll
  for (int a = 0; a < FRA; ++a) {
    const int row = a * 16 + li;
    const int64_t m = m0 + row;
    aval[a] = row < RW && m < M;
    arow[a] = p.A + (aval[a] ? m : 0) * (int64_t)K;
  }
  const uint16_t* brow = p.B + (int64_t)li * K + kq;
  // transposing-read address of this lane in a staged K step (k-major B)
  const int trow = 8 * (lane >> 4) + ((lane >> 2) & 3);
  for (int k0 = 32 * wave; k0 < K; k0 += 512 * U) {
    bf16x8 af[U][FRA];
    bf16x8 bf[BKN ? 1 : U][NJ];
    u32x4 breg[BKN ? U : 1][BL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 512 * u;
      const bool kv = k < K;
#pragma unroll
      for (int a = 0; a < FRA; ++a) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        // ordinary (cacheable) loads: the fused GEMM that follows reads the same
        // rows of X or dY, and streaming loads would push them out of the caches
        if (kv && aval[a]) v = *(const u32x4*)(arow[a] + k + kq);
        af[u][a] = __builtin_bit_cast(bf16x8, v);
      }
      if constexpr (BKN) {
        // rows k .. k+31 of B as 16-byte pieces (piece e: row e/PPR, columns 8*(e%PPR) ..)
#pragma unroll
        for (int i = 0; i < BL; ++i) {
          const int e = lane + 64 * i;
          const int row = e / PPR, c8 = 8 * (e % PPR);
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (kv && e < 32 * PPR && c8 < p.r) v = *(const u32x4*)(p.B + (int64_t)(k + row) * p.bkn + c8);
          breg[u][i] = v;
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (kv) v = *(const u32x4*)(brow + (int64_t)j * 16 * K + k);
          bf[u][j] = __builtin_bit_cast(bf16x8, v);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bf16x8 bk[NJ];
      if constexpr (BKN) {
        // stage the step row-major, then read each 16-column group transposed
#pragma unroll
        for (int i = 0; i < BL; ++i) {
          const int e = lane + 64 * i;
          if (e < 32 * PPR) *(u32x4*)(stage + (e / PPR) * ROWB + 16 * (e % PPR)) = breg[u][i];
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) bk[j] = lds_tr8(stage + trow * ROWB + 2 * (16 * j + 4 * (lane & 3)), ROWB);
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) bk[j] = bf[u][j];
      }
#pragma unroll
      for (int a = 0; a < FRA; ++a)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][a], bk[j], acc[a][j], 0, 0, 0);
    }
  }
  if constexpr (BKN) __syncthreads();  // every wave is done with its stage before the tiles reuse it
  // D[i][jj]: lane holds column jj = lane%16, rows i = 4*(lane/16) + v
#pragma unroll
  for (int a = 0; a < FRA; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = a * 16 + 4 * (lane >> 4) + v;
      if (row < RW) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) red[(wave * RW + row) * RPT + j * 16 + li] = acc[a][j][v];
      }
    }
  __syncthreads();
  for (int e = tid; e < RW * RPT; e += 1024) {
    const int64_t m = m0 + e / RPT;
    if (m >= M) continue;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) sum += red[w * RW * RPT + e];
    const int j = e % RPT;
    if (p.out1 && j < p.r) p.out1[m * p.ld1 + j] = f32_to_bf16(p.alpha1 * sum);
    if (p.out2) p.out2[m * RPT + j] = f32_to_bf16(p.alpha2 * sum);
  }
}


// ---------------------------------------------------------------------------
// NT skinny at rank 16 with a row-major B ([16][K]: G = s dY L2^T), whole K per
// workgroup, with whole-line loads: the same product as k_skinny_nt_rows<16,
// false>.  A 1024-thread workgroup owns 8 rows of A; wave w takes the
// 64-column units w, w + 16, ... of K.  For each unit it loads A as 8 rows x
// 128 bytes (one load, 8 lanes per row) and B as 16 rows x 128 bytes (two
// loads), so every load reads whole 128-byte lines; loads in the MFMA operand
// layout read 64 bytes of each of 16 lines, half of every line they touch.  The
// unit goes through the wave's own LDS area (rows padded to 144 bytes, so the
// 16 rows of a fragment read fall on distinct banks) and is read back as the
// operands of two v_mfma_f32_16x16x32_bf16.  Four units per wave are in flight
// in registers.  The A operand's rows 8..15 repeat rows 0..7; those rows of the
// result are not used.  The 16 wave tiles are added in LDS in wave order.
// (A k-major B is read in whole lines by k_skinny_nt_rows already.)
// ---------------------------------------------------------------------------
constexpr int kLnRow = 144;  // LDS bytes per staged row of a 64-column unit

__global__ __launch_bounds__(1024) void k_skinny_nt_lines(NtArgs p) {
  constexpr int RW = 8, RPT = 16, UU = 4;
  constexpr int SA = RW * kLnRow, SB = RPT * kLnRow;  // A stage: 8 rows; B stage: 16 rows
  constexpr int RED = 16 * RW * RPT * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[RED + 16 * (SA + SB)];
  float* red = (float*)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint8_t* sa = smem + RED + wave * (SA + SB);
  uint8_t* sb = sa + SA;
  const int64_t m0 = (int64_t)blockIdx.x * RW;
  const int64_t M = p.M;
  const int K = p.K;
  // load lanes: row lane/8, 16-byte piece lane%8 of a 128-byte row segment
  const int lr = lane >> 3, lp = lane & 7;
  const bool arow_ok = m0 + lr < M;
  const uint16_t* arow = p.A + (arow_ok ? m0 + lr : 0) * (int64_t)K + 8 * lp;
  // fragment lanes: row li, k offset kq of a 32-column step
  const int li = lane & 15;
  const int kq = (lane >> 4) * 8;
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int kr = 0; kr < K; kr += 1024 * UU) {
    u32x4 ar[UU], br[UU][2];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      const int c0 = kr + 1024 * u + 64 * wave;  // the unit's first column (K % 64 == 0)
      const bool cv = c0 < K;
      ar[u] = (cv && arow_ok) ? *(const u32x4*)(arow + c0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 2; ++i)
        br[u][i] = cv ? *(const u32x4*)(p.B + (int64_t)(8 * i + lr) * K + c0 + 8 * lp) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      if (kr + 1024 * u + 64 * wave >= K) break;
      // stage the unit; the previous unit's reads of this area come first (the
      // LDS operations of one wave complete in order)
      *(u32x4*)(sa + lr * kLnRow + 16 * lp) = ar[u];
#pragma unroll
      for (int i = 0; i < 2; ++i) *(u32x4*)(sb + (8 * i + lr) * kLnRow + 16 * lp) = br[u][i];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 af = *(const bf16x8*)(sa + (li & 7) * kLnRow + 2 * (32 * st + kq));
        const bf16x8 bk = *(const bf16x8*)(sb + li * kLnRow + 2 * (32 * st + kq));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bk, acc, 0, 0, 0);
      }
    }
  }
  // D[i][jj]: lane holds column jj = lane%16, rows i = 4*(lane/16) + v (rows 8..15 unused)
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * (lane >> 4) + v;
    if (row < RW) red[(wave * RW + row) * RPT + li] = acc[v];
  }
  __syncthreads();
  for (int e = tid; e < RW * RPT; e += 1024) {
    const int64_t m = m0 + e / RPT;
    if (m >= M) continue;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) sum += red[w * RW * RPT + e];
    const int j = e % RPT;
    if (p.out1 && j < p.r) p.out1[m * p.ld1 + j] = f32_to_bf16(p.alpha1 * sum);
    if (p.out2) p.out2[m * RPT + j] = f32_to_bf16(p.alpha2 * sum);
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
      if (m + row < m_hi && col < N) v = *(const u32x4*)(p.Q + (m + row) * N + col);
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
// TN skinny, all tokens per workgroup (RP <= 64): the same product as
// k_skinny_tn without a token split.  A workgroup of WAVES = 8 waves owns
// NC = 64 (or 32) columns of Q; with 8 waves rather than 16, each wave takes
// enough chunks at 2048 tokens (64 chunks of 32) for its loads to run ahead
// of its staging and MFMAs.  Wave w takes the 32-token chunks w, w+WAVES, ...: it copies
// each chunk of Q ([32][NC]) and P ([32][RP]) row-major into its own LDS
// area with 16-byte stores (DEPTH chunks ahead in registers) and builds both
// MFMA operands with ds_read_b64_tr_b16, which hands each lane 4 consecutive
// tokens of one column (in each group of 16 lanes, lane 4e+q addresses token
// row e, columns c+4q..c+4q+3, and lane i receives column c+i of the 4 rows).
// LDS rows are padded so the 4 rows of a transposing read fall on distinct
// banks.  The wave tiles are added in LDS in wave order (rounds of four
// slots), so the result does not depend on scheduling.
// ---------------------------------------------------------------------------
template <int RPT, int NC, int WAVES>
struct TnCols {
  static constexpr int NJ = RPT / 16, NG = NC / 16;
  static constexpr int QROW = NC * 2 + (NC == 64 ? 16 : 32);  // LDS bytes per token row
  static constexpr int PROW = RPT * 2 + (RPT * 2 % 64 == 32 ? 16 : (RPT * 2 % 128 == 0 ? 16 : 32));
  static constexpr int QPR = NC / 8, QTL = 64 / QPR, QL = 32 / QTL;     // Q pieces per row, tokens per load, loads
  static constexpr int PPR = RPT / 8, PTL = 64 / PPR, PL = (32 + PTL - 1) / PTL;
  static constexpr int STAGE = 32 * (QROW + PROW);                       // bytes per wave
  // chunks in flight per wave, as many as the register budget allows
  static constexpr int DEPTH = QL + PL <= 6 ? 3 : 2;
  static constexpr int SMEM = WAVES * STAGE > 4 * RPT * NC * 4 ? WAVES * STAGE : 4 * RPT * NC * 4;
};

// One workgroup's share of one product: column band `bid` of `nwg`.
template <int RPT, int NC, int WAVES>
__device__ __forceinline__ void tn_cols_band(const TnArgs& p, int bid, int nwg, uint8_t* smem) {
  using S = TnCols<RPT, NC, WAVES>;
  constexpr int NJ = S::NJ, NG = S::NG, QROW = S::QROW, PROW = S::PROW;
  constexpr int QPR = S::QPR, QTL = S::QTL, QL = S::QL, PPR = S::PPR, PTL = S::PTL, PL = S::PL;
  constexpr int DEPTH = S::DEPTH;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // neighbouring column bands share 128-byte lines of Q: keep them on one XCD
  // (workgroups are dealt to the 8 XCDs round-robin) so they meet in its L2
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int n0 = bid * NC;
  const int64_t M = p.M;
  const int N = p.N;
  uint8_t* qs = smem + wave * S::STAGE;
  uint8_t* ps = qs + 32 * QROW;

  // this lane's pieces of a chunk: Q token QTL*i + lane/QPR, columns 8*(lane%QPR);
  // P token PTL*i + lane/PPR, columns 8*(lane%PPR) (read only below r)
  const int qcol = n0 + 8 * (lane % QPR);
  const bool qok = qcol < N;
  const int pj = 8 * (lane % PPR);
  const bool pok = pj < p.r;
  u32x4 qr[DEPTH][QL], pr[DEPTH][PL];
  const int64_t nchunk = (M + 31) / 32;
  auto load = [&](int slot, int64_t c) {
    const int64_t m0 = c * 32;
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      const int64_t m = m0 + QTL * i + lane / QPR;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      // ordinary (cacheable) loads, as in the NT products: Q is X or dY
      if (c < nchunk && m < M && qok) v = *(const u32x4*)(p.Q + m * N + qcol);
      qr[slot][i] = v;
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int t = PTL * i + lane / PPR;
      const int64_t m = m0 + t;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (c < nchunk && t < 32 && m < M && pok) v = *(const u32x4*)(p.P + m * p.ldp + pj);
      pr[slot][i] = v;
    }
  };
  auto stage = [&](int slot) {
#pragma unroll
    for (int i = 0; i < QL; ++i) *(u32x4*)(qs + (QTL * i + lane / QPR) * QROW + 16 * (lane % QPR)) = qr[slot][i];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int t = PTL * i + lane / PPR;
      if (t < 32) *(u32x4*)(ps + t * PROW + 16 * (lane % PPR)) = pr[slot][i];
    }
  };
  floatx4 acc[NJ][NG];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[j][g] = floatx4{0.f, 0.f, 0.f, 0.f};
  // transposing-read addresses: 16-lane group g16 covers tokens 8*g16 .. +7
  const int g16 = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
  const int trow = 8 * g16 + e;
  auto compute = [&]() {
    bf16x8 bq[NG], ap[NJ];
#pragma unroll
    for (int g = 0; g < NG; ++g) bq[g] = lds_tr8(qs + trow * QROW + 2 * (16 * g + 4 * q), QROW);
#pragma unroll
    for (int j = 0; j < NJ; ++j) ap[j] = lds_tr8(ps + trow * PROW + 2 * (16 * j + 4 * q), PROW);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < NG; ++g) acc[j][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap[j], bq[g], acc[j][g], 0, 0, 0);
  };
  // chunks wave, wave+WAVES, ...: DEPTH in flight in registers while one is multiplied
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load(d, wave + (int64_t)d * WAVES);
  for (int64_t c = wave; c < nchunk; c += (int64_t)DEPTH * WAVES) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int64_t cc = c + (int64_t)d * WAVES;
      if (cc < nchunk) {
        stage(d);
        load(d, cc + (int64_t)DEPTH * WAVES);
        compute();
      }
    }
  }
  // D[i][jj]: lane holds column jj = lane%16 (of column group g), rows i = 4*(lane/16) + v (of j fragment)
  __syncthreads();
  float* slot = (float*)smem;
#pragma unroll
  for (int f = 0; f < WAVES / 4; ++f) {
    if ((wave >> 2) == f) {
      float* mine = slot + (wave & 3) * RPT * NC;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int idx = (j * 16 + 4 * (lane >> 4) + v) * NC + g * 16 + (lane & 15);
            mine[idx] = f == 0 ? acc[j][g][v] : mine[idx] + acc[j][g][v];
          }
    }
    __syncthreads();
  }
  for (int idx = tid; idx < RPT * NC; idx += WAVES * 64) {
    const int j = idx / NC;
    const int n = n0 + idx % NC;
    if (j >= p.r || n >= N) continue;
    const float sum = ((slot[idx] + slot[RPT * NC + idx]) + slot[2 * RPT * NC + idx]) + slot[3 * RPT * NC + idx];
    if (p.trans) p.out[(int64_t)n * p.r + j] = p.alpha * sum;
    else p.out[(int64_t)j * N + n] = p.alpha * sum;
  }
}

// Two TN products in one launch (the first nwg0 workgroups run p0, the rest
// p1), so that two narrow products together fill the chip; nwg1 = 0 runs one.
template <int RPT, int NC, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_skinny_tn_cols(TnArgs p0, TnArgs p1, int nwg0, int nwg1) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[TnCols<RPT, NC, WAVES>::SMEM];
  if ((int)blockIdx.x < nwg0) tn_cols_band<RPT, NC, WAVES>(p0, blockIdx.x, nwg0, smem);
  else tn_cols_band<RPT, NC, WAVES>(p1, blockIdx.x - nwg0, nwg1, smem);
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
  // A launch holds at most 2^32 - 1 work-items, and the whole-K kernel spends
  // 1024 of them on 8 rows.  Each output row depends only on its own row of A,
  // so more rows than kNtLaunchRows run as launches over consecutive row ranges
  // (nt_launch_rows).  Past 2^24 rows the split kernel's K is never split.
  if (a.M > kNtLaunchRows) {
    if (a.ksplit != 1) return hipErrorInvalidValue;
    const int64_t rows = nt_launch_rows(a.M);
    for (int64_t m0 = 0; m0 < a.M; m0 += rows) {
      NtArgs c = a;
      c.A = a.A + m0 * a.K;
      c.M = std::min(rows, a.M - m0);
      if (c.out1) c.out1 = a.out1 + m0 * a.ld1;
      if (c.out2) c.out2 = a.out2 + m0 * RP;
      const hipError_t e = launch_skinny_nt(c, RP, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (a.bkn && !skinny_nt_whole(a.M, RP)) return hipErrorInvalidValue;  // k-major B: whole-K kernel only
  {
    if (skinny_nt_use_whole(a.M, a.K, RP, a.bkn != 0)) {
      const int rw = RP <= 16 ? 8 : (RP <= 32 ? 16 : 32);
      const int64_t nwg = (a.M + rw - 1) / rw;
      const dim3 gr((unsigned)nwg), bl(1024);
#define L_NTR(R)                                                                     \
  if (a.bkn) hipLaunchKernelGGL((k_skinny_nt_rows<R, true>), gr, bl, 0, st, a);      \
  else hipLaunchKernelGGL((k_skinny_nt_rows<R, false>), gr, bl, 0, st, a);
      switch (RP) {
        case 16:
          if (a.bkn) hipLaunchKernelGGL((k_skinny_nt_rows<16, true>), gr, bl, 0, st, a);
          else hipLaunchKernelGGL(k_skinny_nt_lines, gr, bl, 0, st, a);
          break;
        case 32: L_NTR(32) break;
        case 48: L_NTR(48) break;
        default: L_NTR(64) break;
      }
#undef L_NTR
      return hipGetLastError();
    }
  }
  const int64_t mblocks = (a.M + 63) / 64;
  const dim3 gr((unsigned)(mblocks * a.ksplit)), bl(256);
#define L_NT(R) hipLaunchKernelGGL(k_skinny_nt<R>, gr, bl, 0, st, a)
  NF4K_RP_SWITCH(RP, L_NT)
#undef L_NT
  return hipGetLastError();
}

// One TN product, or two (b != NULL, same M) in one launch when both take the
// all-token kernel; otherwise the split kernel runs each.
hipError_t launch_skinny_tn2(const TnArgs& a, const TnArgs* b, int RP, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  // all tokens per workgroup when the rank is small: 64 columns each (each load
  // of Q reads whole 128-byte lines), or 32 when 64-column bands would leave
  // fewer than 192 workgroups for the 256 CUs (skinny_tn_band)
  if (skinny_tn_whole(a.M, RP)) {
    const bool wide = skinny_tn_band(a.N, b ? b->N : 0) == 64;
    const int nc = wide ? 64 : 32;
    const int nwg0 = (a.N + nc - 1) / nc, nwg1 = b ? (b->N + nc - 1) / nc : 0;
    const TnArgs& a1 = b ? *b : a;
    const dim3 gr((unsigned)(nwg0 + nwg1)), bl(512);
#define L_TNC(R)                                                                                          \
  if (wide) hipLaunchKernelGGL((k_skinny_tn_cols<R, 64, 8>), gr, bl, 0, st, a, a1, nwg0, nwg1); \
  else hipLaunchKernelGGL((k_skinny_tn_cols<R, 32, 8>), gr, bl, 0, st, a, a1, nwg0, nwg1);
    switch (RP) {
      case 16: L_TNC(16) break;
      case 32: L_TNC(32) break;
      case 48: L_TNC(48) break;
      default: L_TNC(64) break;
    }
#undef L_TNC
    return hipGetLastError();
  }
  for (const TnArgs* t : {&a, b}) {
    if (!t) continue;
    const int nblocks = (t->N + 63) / 64;
    const dim3 gr((unsigned)(nblocks * t->msplit)), bl(256);
#define L_TN(R) hipLaunchKernelGGL(k_skinny_tn<R>, gr, bl, 0, st, *t)
    NF4K_RP_SWITCH(RP, L_TN)
#undef L_TN
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_skinny_tn(const TnArgs& a, int RP, hipStream_t st) { return launch_skinny_tn2(a, nullptr, RP, st); }

}  // namespace nf4k
