// NF4 quantize / dequantize / reconstruction-error / top-K kernels (gfx950).
//
// The weight is a row-major fp32 [rows][cols] array with cols % 64 == 0, so
// block b is the 64 consecutive floats starting at element 64*b and no block
// crosses a row.  One workgroup (256 threads, 4 wave64s) owns one group of 256
// consecutive blocks (16,384 weights): each wave streams 64 blocks in 8
// rounds of 8 blocks; in a round the 8 lanes of a half DPP row hold one block,
// two float4 each (elements 4l..4l+3 and 32+4l..32+4l+3 of lane l), so each of
// the round's two loads reads whole 128-byte lines, the block absmax is a
// 3-step DPP max inside the half row, the per-block setup is paid once per 8
// weights of a lane, and the double-quantization group max needs no second
// pass over HBM.
//
// Format ("QLoRA: How to fine-tune large language models with less memory",
// sections "1. NormalFloat" and "2. Double quantization"): 4-bit codes, two
// per byte (even element in the low nibble), one fp32 absmax per 64 weights,
// or one 8-bit scale code per block plus an fp32 step per 256 blocks.
#include "common.hpp"
#include "launch.hpp"

namespace nf4k {

// ---------------------------------------------------------------------------
// quantize
// ---------------------------------------------------------------------------
constexpr uint32_t kRsrcFlags = 0x00020000u;  // raw buffer, gfx9-family dword3
constexpr int kNT = 2;                        // cache policy: streaming (nt)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcFlags);
}

// The 8 rounds of one wave: round i covers blocks lb = wave*64 + 8i + sub of
// the group (sub = lane/8); lane l8 = lane%8 holds quads l8 and 8 + l8 of its
// block (elements 4*l8 .. +3 in v[i][0], 32 + 4*l8 .. +3 in v[i][1]).  Reads
// past the group's last block return zero.
__device__ __forceinline__ void load_group(__amdgpu_buffer_rsrc_t wr, int wave, int sub, int l8, floatx4 (&v)[8][2]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lb = wave * 64 + 8 * i + sub;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      v[i][h] = __builtin_bit_cast(floatx4,
                                   __builtin_amdgcn_raw_buffer_load_b128(wr, (lb * 64 + (8 * h + l8) * 4) * 4, 0, kNT));
  }
}

// Round i of load_group alone.
__device__ __forceinline__ void load_round(__amdgpu_buffer_rsrc_t wr, int wave, int sub, int l8, int i,
                                           floatx4 (&v)[8][2]) {
  const int lb = wave * 64 + 8 * i + sub;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    v[i][h] = __builtin_bit_cast(floatx4,
                                 __builtin_amdgcn_raw_buffer_load_b128(wr, (lb * 64 + (8 * h + l8) * 4) * 4, 0, kNT));
}
// Rounds of loads kept in flight ahead of the round being encoded, when a
// wave encodes its rounds as they arrive: 4 rounds (128 KB per CU) are more
// than the memory system needs in flight, and the last round to arrive then
// leaves one round of work after it instead of eight.
constexpr int kAhead = 4;

// Encoder table in LDS, one 16-byte entry per bucket (see NF4Enc):
// {fp64 bound, code (quantize) or value bits (error) below / above the bound}.
struct EncEntry {
  double bound;
  uint32_t lo, hi;
};
template <bool VALUES>
__device__ __forceinline__ void enc_to_lds(const NF4Enc& e, EncEntry* t, int tid) {
  if (tid < e.nb) {
    EncEntry x;
    x.bound = e.bound[tid];
    x.lo = VALUES ? __builtin_bit_cast(uint32_t, e.qlo[tid]) : e.code_lo[tid];
    x.hi = VALUES ? __builtin_bit_cast(uint32_t, e.qhi[tid]) : e.code_hi[tid];
    t[tid] = x;
  }
}

// Per-block setup of the division-free encoder: m' = m (or 1 for an all-zero
// block, whose weights are all +-0 and take the code of 0), an approximate
// 1/m' and a power-of-two prescale keeping that reciprocal in the normal range.
struct BlockEnc {
  float s, y;
  double md;
};
__device__ __forceinline__ BlockEnc block_enc(float m) {
  BlockEnc b;
  const float mp = (m > 0.f) ? m : 1.f;
  b.s = (mp < 0x1p-64f) ? 0x1p64f : ((mp > 0x1p64f) ? 0x1p-64f : 1.f);
  b.y = __builtin_amdgcn_rcpf(mp * b.s);
  b.md = (double)mp;
  return b;
}
// x > t for the threshold t of the bucket of x = fl32(w / m'), decided
// exactly; returns the table entry through `en`.
__device__ __forceinline__ bool above(float w, const BlockEnc& b, float bscale, float boffset, const EncEntry* tab,
                                      EncEntry& en) {
  // xq is within 2e-7 of w / m' and |xq| <= 1 + 2e-7, so k is in 0 .. nb-1
  // (a NaN weight converts to bucket 0)
  const float xq = (w * b.s) * b.y;
  const uint32_t k = (uint32_t)__builtin_fmaf(xq, bscale, boffset);
  en = tab[k];
  return fma(-en.bound, b.md, (double)w) > 0.0;
}

// codes of 4 weights of a block, packed into 16 bits
__device__ __forceinline__ uint32_t encode4(floatx4 v, const BlockEnc& b, float bscale, float boffset,
                                            const EncEntry* tab) {
  const float w[4] = {v.x, v.y, v.z, v.w};
  uint32_t p = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    EncEntry en;
    const bool up = above(w[e], b, bscale, boffset, tab, en);
    p |= (up ? en.hi : en.lo) << (4 * e);
  }
  return p;
}

// absmax of a block held by 8 lanes (two float4 each): an integer max of the
// |w| bit patterns, then a max across the half DPP row
__device__ __forceinline__ float block_absmax(const floatx4 (&v)[2]) {
  const u32x4 a = __builtin_bit_cast(u32x4, v[0]) & 0x7FFFFFFFu;
  const u32x4 b = __builtin_bit_cast(u32x4, v[1]) & 0x7FFFFFFFu;
  uint32_t x = max(max(max(a.x, a.y), max(a.z, a.w)), max(max(b.x, b.y), max(b.z, b.w)));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, true));  // row_half_mirror
  return __builtin_bit_cast(float, x);
}

// max over the 256 threads of the workgroup (every thread gets it)
__device__ __forceinline__ float group_max(float gm, int lane, int wave) {
  __shared__ float red[4];
  gm = fmaxf(gm, __shfl_xor(gm, 16));
  gm = fmaxf(gm, __shfl_xor(gm, 32));
  if (lane == 0) red[wave] = gm;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Outputs of one quantization stage (absmax: fp32 scales; c8/dqs: 8-bit scales and steps).
struct QStage {
  uint8_t* codes;
  float* absmax;
  uint8_t* c8;
  float* dqs;
};

// One weight's terms of the error, added to the running sums: the decoded
// value wh = fl32(table[c] * sc) is fp32 as the format defines; the difference
// of the two fp32 values and both squares are fp64 (squares of fp32 weights can
// leave the fp32 range), each square added with one fused multiply-add.  Both error
// kernels add the weights in the same order (round, quad, element), so their
// per-group partial sums agree bit for bit.
__device__ __forceinline__ void error_term(float w, float wh, double& dsum, double& wsum) {
  const double wd = (double)w;
  const double d = wd - (double)wh;
  dsum = fma(d, d, dsum);
  wsum = fma(wd, wd, wsum);
}

// error_term over one quad (4 weights of one block) of the one-pass kernel
__device__ __forceinline__ void error_round(floatx4 v, uint32_t packed, float sc, const float* tab, double& dsum,
                                            double& wsum) {
  const float w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) error_term(w4[e], tab[(packed >> (4 * e)) & 15u] * sc, dsum, wsum);
  // materialise the sums here: otherwise the compiler sinks every round's
  // error arithmetic past the group-max barrier and keeps all 16 rounds live
  asm volatile("" : "+v"(dsum), "+v"(wsum));
}

// One group's partial sums {sum (w - w_hat)^2, sum w^2} to part[2g], part[2g+1]:
// xor tree inside each wave, then waves 0..3 in order.
__device__ __forceinline__ void error_group_out(double dsum, double wsum, int lane, int wave, int tid, int64_t g,
                                                double* __restrict__ part) {
  __shared__ double redd[2][4];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    dsum += __shfl_xor(dsum, o);
    wsum += __shfl_xor(wsum, o);
  }
  if (lane == 0) {
    redd[0][wave] = dsum;
    redd[1][wave] = wsum;
  }
  __syncthreads();
  if (tid == 0) {
    part[2 * g + 0] = ((redd[0][0] + redd[0][1]) + redd[0][2]) + redd[0][3];
    part[2 * g + 1] = ((redd[1][0] + redd[1][1]) + redd[1][2]) + redd[1][3];
  }
}

// ERR: 0 = quantize only; 1 = also the reconstruction error with the plain
// block absmax as scale; 2 = with the double-quantized scales (DQ only).  The
// error's per-group partials (as k_error_partial writes them) go to `part`.
template <bool DQ, bool RES, int ERR>
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ W, int64_t nblocks, QStage o1, QStage o2,
                                                  double* __restrict__ part, NF4Enc enc, NF4Consts cst) {
  static_assert(ERR == 0 || !RES, "the error pass covers one stage");
  static_assert(ERR != 2 || DQ, "the double-quantized error needs the group step");
  __shared__ EncEntry etab[kMaxBuckets];
  __shared__ float tab[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane >> 3;
  const int l8 = lane & 7;
  const int64_t g = blockIdx.x;
  const int64_t gb0 = g * 256;
  const uint32_t nb = (uint32_t)min((int64_t)256, nblocks - gb0);  // blocks in this group
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W + gb0 * 64, nb * 256);
  enc_to_lds<false>(enc, etab, tid);
  if ((RES || ERR) && tid < 16) tab[tid] = cst.table[tid];

  // PIPE: the rounds are encoded as they arrive, kAhead rounds of loads in
  // flight ahead of the one being encoded (the error with 8-bit scales and the
  // residual stage need every block of the group first)
  constexpr bool PIPE = ERR != 2 && !RES;
  floatx4 v[8][2];
  if constexpr (PIPE) {
#pragma unroll
    for (int i = 0; i < kAhead; ++i) load_round(wr, wave, sub, l8, i, v);
  } else {
    load_group(wr, wave, sub, l8, v);
  }
  __syncthreads();  // encoder tables

  float amax[8];
  uint32_t packed[8];  // round i: quad l8's codes in bits 0..15, quad 8 + l8's in 16..31
  double dsum = 0.0, wsum = 0.0;
  // lane l8 of half row `sub` owns the block of round l8: lb = wave*64 + 8*l8 + sub
  const int mylb = wave * 64 + 8 * l8 + sub;
  // (absmax bit patterns are non-negative integers: an integer max over the
  // rounds, the others masked to 0, picks round l8's value bit for bit)
  auto my_amax = [&]() -> float {
    uint32_t mb = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) mb = max(mb, (l8 == i) ? __builtin_bit_cast(uint32_t, amax[i]) : 0u);
    return __builtin_bit_cast(float, mb);
  };
  // double-quantization step of the group, S = fl32(max absmax / 255): the 8
  // rounds of this lane's half row, then the other half rows, then waves
  auto group_step = [&](float mine) -> float {
    float gm = mine;
    gm = fmaxf(gm, __shfl_xor(gm, 1));
    gm = fmaxf(gm, __shfl_xor(gm, 2));
    gm = fmaxf(gm, __shfl_xor(gm, 4));
    gm = fmaxf(gm, __shfl_xor(gm, 8));
    return group_max(gm, lane, wave) / 255.0f;
  };
  // one stage over v: codes, block scales and (DQ) the group's 8-bit scales;
  // returns the group step S (0 without double quantization)
  auto stage = [&](const QStage& o) -> float {
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(o.codes + gb0 * 32, nb * 32);
    float S = 0.f;
    if constexpr (ERR == 2) {
      // the error with 8-bit scales needs S before any round: block maxima first
#pragma unroll
      for (int i = 0; i < 8; ++i) amax[i] = block_absmax(v[i]);
      S = group_step(my_amax());
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // with the error, one round at a time keeps the fp64 temporaries short-lived
      if constexpr (ERR != 0 || PIPE) __builtin_amdgcn_sched_barrier(0);
      if constexpr (PIPE) {
        if (i + kAhead < 8) load_round(wr, wave, sub, l8, i + kAhead, v);
        __builtin_amdgcn_sched_barrier(0);
      }
      const float m = (ERR == 2) ? amax[i] : block_absmax(v[i]);
      amax[i] = m;
      const BlockEnc be = block_enc(m);
      packed[i] = encode4(v[i][0], be, enc.bscale, enc.boffset, etab) |
                  (encode4(v[i][1], be, enc.bscale, enc.boffset, etab) << 16);
      if constexpr (ERR != 0) {
        const float sc = (ERR == 1) ? m : ((S > 0.f) ? fminf(255.f, rintf(m / S)) * S : 0.f);
        error_round(v[i][0], packed[i] & 0xFFFFu, sc, tab, dsum, wsum);
        error_round(v[i][1], packed[i] >> 16, sc, tab, dsum, wsum);
      }
      const int lb = wave * 64 + 8 * i + sub;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(packed[i] >> (16 * h)), cr, lb * 32 + (8 * h + l8) * 2,
                                              0, kNT);
    }
    const float mine = my_amax();
    if constexpr (!DQ) {
      const __amdgpu_buffer_rsrc_t ar = make_rsrc(o.absmax + gb0, nb * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, mine), ar, mylb * 4, 0, 0);
      return 0.f;
    } else {
      if constexpr (ERR != 2) S = group_step(mine);
      if (tid == 0) o.dqs[g] = S;
      const uint32_t q = (S > 0.f) ? (uint32_t)fminf(255.f, rintf(mine / S)) : 0u;
      const __amdgpu_buffer_rsrc_t qr = make_rsrc(o.c8 + gb0, nb);
      __builtin_amdgcn_raw_buffer_store_b8((unsigned char)q, qr, mylb, 0, 0);
      return S;
    }
  };
  const float S1 = stage(o1);
  if constexpr (ERR != 0) error_group_out(dsum, wsum, lane, wave, tid, g, part);
  if constexpr (RES) {
    // residual of the first stage, in place: r = fl32(w - fl32(table[c] * a_hat))
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float sc = amax[i];
      if constexpr (DQ) sc = (S1 > 0.f) ? fminf(255.f, rintf(amax[i] / S1)) * S1 : 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t pk = packed[i] >> (16 * h);
        v[i][h].x = v[i][h].x - tab[pk & 15u] * sc;
        v[i][h].y = v[i][h].y - tab[(pk >> 4) & 15u] * sc;
        v[i][h].z = v[i][h].z - tab[(pk >> 8) & 15u] * sc;
        v[i][h].w = v[i][h].w - tab[(pk >> 12) & 15u] * sc;
      }
    }
    __syncthreads();  // the first stage's group-max slots are read before the second stage reuses them
    stage(o2);
  }
}

// ---------------------------------------------------------------------------
// dequantize: each thread expands code dwords (8 weights of one block each),
// four per round for bf16 output and one for fp32
// ---------------------------------------------------------------------------
constexpr int kDequantWordsBf16 = 4;  // code words per thread and round, bf16 output

template <bool DQ, bool BF16, bool RES>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes,
                                                    const void* __restrict__ absmax,
                                                    const float* __restrict__ dqs,
                                                    const uint8_t* __restrict__ codes2,
                                                    const void* __restrict__ absmax2,
                                                    const float* __restrict__ dqs2,
                                                    int64_t nwords, void* __restrict__ out,
                                                    NF4Consts cst) {
  __shared__ float tab[16];
  if (threadIdx.x < 16) tab[threadIdx.x] = cst.table[threadIdx.x];
  __syncthreads();
  auto scale = [&](const void* am, const float* dq, int64_t blk) -> float {
    if constexpr (DQ) return (float)((const uint8_t*)am)[blk] * dq[blk >> 8];
    else return ((const float*)am)[blk];
  };
  if constexpr (BF16) {
    // A workgroup takes 256 U consecutive code words per round: word
    // base + 256 j + threadIdx.x for j < U, so each load and store instruction
    // of a wave covers one contiguous span.  All U words and their scales are
    // loaded before the first is used: the code stream is small next to the
    // output, and only loads in flight keep it moving.
    constexpr int U = kDequantWordsBf16;
    const int64_t stride = (int64_t)gridDim.x * (256 * U);
    for (int64_t base = (int64_t)blockIdx.x * (256 * U); base < nwords; base += stride) {
      uint32_t w[U], w2[U];
      float sc[U], sc2[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t t = base + 256 * j + threadIdx.x;
        const bool in = t < nwords;
        w[j] = in ? __builtin_nontemporal_load((const uint32_t*)codes + t) : 0u;
        if constexpr (RES) w2[j] = in ? __builtin_nontemporal_load((const uint32_t*)codes2 + t) : 0u;
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t t = base + 256 * j + threadIdx.x;
        const bool in = t < nwords;
        sc[j] = in ? scale(absmax, dqs, t >> 3) : 0.f;
        if constexpr (RES) sc2[j] = in ? scale(absmax2, dqs2, t >> 3) : 0.f;
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t t = base + 256 * j + threadIdx.x;
        if (t >= nwords) break;
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = tab[(w[j] >> (4 * e)) & 15u] * sc[j];
        if constexpr (RES) {
          // second stage: w_hat = fl32(w_hat1 + w_hat2)
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = f[e] + tab[(w2[j] >> (4 * e)) & 15u] * sc2[j];
        }
        const u32x4 o = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                         pack_bf16x2(f[6], f[7])};
        __builtin_nontemporal_store(o, (u32x4*)out + t);
      }
    }
  } else {
    // fp32 output: one word per thread and round.  Each word is two 16-byte
    // stores that interleave within a line; with more words in flight this
    // pass got slower (4.4 -> 3.0 TB/s at 45 M weights).
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nwords; t += stride) {
      const uint32_t w = __builtin_nontemporal_load((const uint32_t*)codes + t);
      const float sc = scale(absmax, dqs, t >> 3);
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = tab[(w >> (4 * e)) & 15u] * sc;
      if constexpr (RES) {
        const uint32_t w2 = __builtin_nontemporal_load((const uint32_t*)codes2 + t);
        const float sc2 = scale(absmax2, dqs2, t >> 3);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = f[e] + tab[(w2 >> (4 * e)) & 15u] * sc2;
      }
      floatx4* o = (floatx4*)out + 2 * t;
      __builtin_nontemporal_store((floatx4{f[0], f[1], f[2], f[3]}), o);
      __builtin_nontemporal_store((floatx4{f[4], f[5], f[6], f[7]}), o + 1);
    }
  }
}

// ---------------------------------------------------------------------------
// reconstruction error, stage 1: per-group fp64 partial sums of (w - w_hat)^2
// and w^2 (encode/decode in fp32 as the format defines, differences and
// squares in fp64).  Same block/group mapping as k_quantize; the weights stay in
// registers between the absmax, group-max and encode/decode steps.
// ---------------------------------------------------------------------------
// Up to kErrBatch linears of one batched error pass, passed by value as a
// kernel argument (1.6 KB): W and its block count per linear, and the first
// partial slot of each linear relative to the launch (g0[n] = slots in all).
struct ErrBatch {
  const float* W[kErrBatch];
  int64_t nblocks[kErrBatch];
  int64_t g0[kErrBatch + 1];
  int32_t n;
};

// One group g of 256 blocks of W: its partial sums go to part[2 slot],
// part[2 slot + 1].  The encoder table `etab` is filled by the caller before
// the first group; the group's first barrier publishes it.
template <bool DQ>
__device__ __forceinline__ void error_partial_group(const float* __restrict__ W, int64_t nblocks, int64_t g,
                                                    int64_t slot, double* __restrict__ part, const NF4Enc& enc,
                                                    const EncEntry* etab) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane >> 3;
  const int l8 = lane & 7;
  const int64_t gb0 = g * 256;
  const uint32_t nb = (uint32_t)min((int64_t)256, nblocks - gb0);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W + gb0 * 64, nb * 256);

  floatx4 v[8][2];
  load_group(wr, wave, sub, l8, v);
  float amax[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) amax[i] = block_absmax(v[i]);
  float S = 0.f;
  if constexpr (DQ) {
    // the 8 rounds of this half row, the other half rows of the wave, then waves
    float gm = amax[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) gm = fmaxf(gm, amax[i]);
    gm = fmaxf(gm, __shfl_xor(gm, 8));
    S = group_max(gm, lane, wave) / 255.0f;  // its barrier also publishes the encoder table
  } else {
    __syncthreads();  // publishes the encoder table
  }

  // dequantization scale of each round's block
  float sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sc[i] = amax[i];
    if constexpr (DQ) sc[i] = (S > 0.f) ? fminf(255.f, rintf(amax[i] / S)) * S : 0.f;
  }
  double dsum = 0.0, wsum = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // one round at a time, its two quads in order, each quad's weights in order
    // (the order of the one-pass quantize + error kernel)
    __builtin_amdgcn_sched_barrier(0);
    const BlockEnc be = block_enc(amax[i]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float w4[4] = {v[i][h].x, v[i][h].y, v[i][h].z, v[i][h].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        EncEntry en;
        const bool up = above(w4[e], be, enc.bscale, enc.boffset, etab, en);
        error_term(w4[e], __builtin_bit_cast(float, up ? en.hi : en.lo) * sc[i], dsum, wsum);
      }
    }
  }
  error_group_out(dsum, wsum, lane, wave, tid, slot, part);
}

template <bool DQ>
__global__ __launch_bounds__(256) void k_error_partial(const float* __restrict__ W, int64_t nblocks,
                                                       double* __restrict__ part, NF4Enc enc) {
  __shared__ EncEntry etab[kMaxBuckets];
  enc_to_lds<true>(enc, etab, threadIdx.x);
  error_partial_group<DQ>(W, nblocks, blockIdx.x, blockIdx.x, part, enc, etab);
}

// The same partial sums for up to kErrBatch linears in one launch, one
// workgroup per group.  The linears' groups are numbered one after another
// (linear i owns slots b.g0[i] .. b.g0[i + 1] - 1); lane l of each wave
// compares slot g with b.g0[l + 1], and the count of the linears that end at
// or before g is the linear that owns it.
template <bool DQ>
__global__ __launch_bounds__(256) void k_error_partial_batch(ErrBatch b, double* __restrict__ part, NF4Enc enc) {
  __shared__ EncEntry etab[kMaxBuckets];
  enc_to_lds<true>(enc, etab, threadIdx.x);
  const int64_t g = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const bool done = lane < b.n && b.g0[lane + 1] <= g;
  const int i = __builtin_amdgcn_readfirstlane(__builtin_popcountll(__ballot(done)));
  error_partial_group<DQ>(b.W[i], b.nblocks[i], g - b.g0[i], g, part, enc, etab);
}

// stage 2: one workgroup sums a linear's per-group partials in a fixed order
// and writes its error.
__device__ __forceinline__ void error_final_sum(const double* __restrict__ part, int64_t ngroups,
                                                double* __restrict__ err) {
  __shared__ double sd[256], sw[256];
  const int tid = threadIdx.x;
  // thread t adds groups t, t + 256, t + 512, ... in that order; the loads of
  // four consecutive terms are issued together (a missing term adds +0.0,
  // which leaves the non-negative sums unchanged)
  double d = 0.0, w = 0.0;
  for (int64_t g0 = tid; g0 < ngroups; g0 += 1024) {
    double2 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t g = g0 + 256 * u;
      x[u] = (g < ngroups) ? ((const double2*)part)[g] : double2{0.0, 0.0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      d += x[u].x;
      w += x[u].y;
    }
  }
  sd[tid] = d;
  sw[tid] = w;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      sd[tid] += sd[tid + s];
      sw[tid] += sw[tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) err[0] = (sw[0] > 0.0) ? sqrt(sd[0]) / sqrt(sw[0]) : 0.0;
}

__global__ __launch_bounds__(256) void k_error_final(const double* __restrict__ part, int64_t ngroups,
                                                     double* __restrict__ err) {
  error_final_sum(part, ngroups, err);
}

// one workgroup per linear of a batch
__global__ __launch_bounds__(256) void k_error_final_batch(ErrBatch b, const double* __restrict__ part,
                                                           double* __restrict__ err) {
  const int i = blockIdx.x;
  error_final_sum(part + 2 * b.g0[i], b.g0[i + 1] - b.g0[i], err + i);
}

// ---------------------------------------------------------------------------
// top-K by rank counting: rank(i) = #{j : j beats i}.  j beats i when e_j is
// NaN and e_i is not, or both are NaN and j < i, or both are numbers and
// e_j > e_i or (e_j == e_i and j < i): a total order in which a NaN error (a
// weight with an Inf or NaN in it) ranks above every number, so every rank
// 0 .. n-1 is taken exactly once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool topk_beats(double ej, int j, double ei, int i) {
  const bool nj = ej != ej, ni = ei != ei;
  if (nj != ni) return nj;
  if (nj || ej == ei) return j < i;
  return ej > ei;
}

__global__ __launch_bounds__(1024) void k_topk(const double* __restrict__ e, int n, int k,
                                               int* __restrict__ idx) {
  __shared__ double tile[1024];
  if (n <= 1024) {
    // one tile: every error is read from global memory once
    const int i = threadIdx.x;
    if (i < n) tile[i] = e[i];
    __syncthreads();
    if (i < n) {
      const double ei = tile[i];
      int rank = 0;
      for (int j = 0; j < n; ++j) rank += topk_beats(tile[j], j, ei, i) ? 1 : 0;
      if (rank < k) idx[rank] = i;
    }
    return;
  }
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const double ei = (i < n) ? e[i] : 0.0;
    int rank = 0;
    for (int t0 = 0; t0 < n; t0 += 1024) {
      __syncthreads();
      if (t0 + (int)threadIdx.x < n) tile[threadIdx.x] = e[t0 + threadIdx.x];
      __syncthreads();
      const int lim = min(1024, n - t0);
      for (int jj = 0; jj < lim; ++jj) rank += topk_beats(tile[jj], t0 + jj, ei, i) ? 1 : 0;
    }
    if (i < n && rank < k) idx[rank] = i;
  }
}

// ---------------------------------------------------------------------------
// the checked mode's scan: flag = 1 when any weight is an infinity or a NaN
// (exponent bits all ones).  The flag is cleared by k_flag_clear first; every
// thread that finds one stores 1 (all stores write the same value).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_flag_clear(int* __restrict__ flag) {
  if (threadIdx.x == 0) flag[0] = 0;
}

__global__ __launch_bounds__(256) void k_check_finite(const float* __restrict__ W, int64_t count,
                                                      int* __restrict__ flag) {
  const int64_t n4 = count >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bool bad = false;
  for (int64_t t = t0; t < n4; t += stride) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)W + t);
    const u32x4 ex = v & 0x7F800000u;
    bad |= (ex.x == 0x7F800000u) | (ex.y == 0x7F800000u) | (ex.z == 0x7F800000u) | (ex.w == 0x7F800000u);
  }
  // the last count % 4 weights
  if (t0 < (count & 3)) {
    const uint32_t b = __builtin_bit_cast(uint32_t, W[n4 * 4 + t0]);
    bad |= (b & 0x7F800000u) == 0x7F800000u;
  }
  if (bad) flag[0] = 1;
}

// ---------------------------------------------------------------------------
// host-side launchers (called from the C ABI layer)
// ---------------------------------------------------------------------------
hipError_t launch_quantize(const float* W, int64_t nblocks, bool dq, uint8_t* codes, void* absmax, float* dqs,
                           uint8_t* codes2, void* absmax2, float* dqs2, const NF4Enc& e, const NF4Consts& c,
                           hipStream_t st) {
  const int64_t ng = (nblocks + 255) / 256;
  if (ng == 0) return hipSuccess;
  if (ng > kMaxLaunchGroups) return hipErrorInvalidValue;
  QStage o1{codes, dq ? nullptr : (float*)absmax, dq ? (uint8_t*)absmax : nullptr, dqs};
  QStage o2{codes2, dq ? nullptr : (float*)absmax2, dq ? (uint8_t*)absmax2 : nullptr, dqs2};
  const dim3 gr((unsigned)ng), bl(256);
  double* const np = nullptr;
  if (codes2) {
    if (dq) hipLaunchKernelGGL((k_quantize<true, true, 0>), gr, bl, 0, st, W, nblocks, o1, o2, np, e, c);
    else hipLaunchKernelGGL((k_quantize<false, true, 0>), gr, bl, 0, st, W, nblocks, o1, o2, np, e, c);
  } else {
    if (dq) hipLaunchKernelGGL((k_quantize<true, false, 0>), gr, bl, 0, st, W, nblocks, o1, o2, np, e, c);
    else hipLaunchKernelGGL((k_quantize<false, false, 0>), gr, bl, 0, st, W, nblocks, o1, o2, np, e, c);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_error(const float* W, int64_t nblocks, bool dq, uint8_t* codes, void* absmax, float* dqs,
                                 bool err_dq, double* part, double* err, const NF4Enc& e, const NF4Consts& c,
                                 hipStream_t st) {
  const int64_t ng = (nblocks + 255) / 256;
  if (err_dq && !dq) return hipErrorInvalidValue;
  if (ng > kMaxLaunchGroups) return hipErrorInvalidValue;
  if (ng > 0) {
    QStage o1{codes, dq ? nullptr : (float*)absmax, dq ? (uint8_t*)absmax : nullptr, dqs};
    const QStage o2{nullptr, nullptr, nullptr, nullptr};
    const dim3 gr((unsigned)ng), bl(256);
    if (err_dq) hipLaunchKernelGGL((k_quantize<true, false, 2>), gr, bl, 0, st, W, nblocks, o1, o2, part, e, c);
    else if (dq) hipLaunchKernelGGL((k_quantize<true, false, 1>), gr, bl, 0, st, W, nblocks, o1, o2, part, e, c);
    else hipLaunchKernelGGL((k_quantize<false, false, 1>), gr, bl, 0, st, W, nblocks, o1, o2, part, e, c);
    hipError_t r = hipGetLastError();
    if (r != hipSuccess) return r;
  }
  hipLaunchKernelGGL(k_error_final, dim3(1), dim3(256), 0, st, part, ng, err);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const void* absmax, const float* dqs, const uint8_t* codes2,
                             const void* absmax2, const float* dqs2, int64_t nweights, bool dq, bool bf16, void* out,
                             const NF4Consts& c, hipStream_t st) {
  const int64_t nwords = nweights / 8;
  if (nwords == 0) return hipSuccess;
  const int64_t per = bf16 ? 256 * kDequantWordsBf16 : 256;
  int64_t blocks = (nwords + per - 1) / per;
  const int64_t cap = bf16 ? 256 * 32 : 256 * 64;  // 32 or 64 workgroups per CU, then a grid-stride loop
  if (blocks > cap) blocks = cap;
  const dim3 gr((unsigned)blocks), bl(256);
#define NF4K_DEQ(D, B, R)                                                                                         \
  hipLaunchKernelGGL((k_dequantize<D, B, R>), gr, bl, 0, st, codes, absmax, dqs, codes2, absmax2, dqs2, nwords, \
                     out, c)
  const bool res = codes2 != nullptr;
  if (res) {
    if (dq && bf16) NF4K_DEQ(true, true, true);
    else if (dq) NF4K_DEQ(true, false, true);
    else if (bf16) NF4K_DEQ(false, true, true);
    else NF4K_DEQ(false, false, true);
  } else {
    if (dq && bf16) NF4K_DEQ(true, true, false);
    else if (dq) NF4K_DEQ(true, false, false);
    else if (bf16) NF4K_DEQ(false, true, false);
    else NF4K_DEQ(false, false, false);
  }
#undef NF4K_DEQ
  return hipGetLastError();
}

hipError_t launch_error(const float* W, int64_t nblocks, bool dq, double* part, double* err,
                        const NF4Enc& c, hipStream_t st) {
  const int64_t ng = (nblocks + 255) / 256;
  if (ng > kMaxLaunchGroups) return hipErrorInvalidValue;
  if (ng > 0) {
    if (dq) {
      hipLaunchKernelGGL(k_error_partial<true>, dim3((unsigned)ng), dim3(256), 0, st, W, nblocks, part, c);
    } else {
      hipLaunchKernelGGL(k_error_partial<false>, dim3((unsigned)ng), dim3(256), 0, st, W, nblocks, part, c);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_error_final, dim3(1), dim3(256), 0, st, part, ng, err);
  return hipGetLastError();
}

hipError_t launch_error_batch(const float* const* W, const int64_t* rows, const int64_t* cols, int32_t n, bool dq,
                              double* part, double* err, const NF4Enc& c, hipStream_t st) {
  int64_t slot = 0;  // first partial slot of the chunk
  for (int32_t c0 = 0; c0 < n;) {
    ErrBatch b{};
    b.n = error_batch_chunk(rows, cols, n, c0, b.g0);
    if (b.n == 0) return hipErrorInvalidValue;  // one linear beyond kMaxLaunchGroups groups
    for (int i = 0; i < b.n; ++i) {
      b.W[i] = W[c0 + i];
      b.nblocks[i] = rows[c0 + i] * cols[c0 + i] / 64;
    }
    const int64_t slots = b.g0[b.n];
    if (slots > 0) {
      const dim3 grid((unsigned)slots);
      if (dq) hipLaunchKernelGGL(k_error_partial_batch<true>, grid, dim3(256), 0, st, b, part + 2 * slot, c);
      else hipLaunchKernelGGL(k_error_partial_batch<false>, grid, dim3(256), 0, st, b, part + 2 * slot, c);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_error_final_batch, dim3((unsigned)b.n), dim3(256), 0, st, b, part + 2 * slot, err + c0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    slot += slots;
    c0 += b.n;
  }
  return hipSuccess;
}

hipError_t launch_check_finite(const float* W, int64_t count, int* flag_dev, hipStream_t st) {
  hipLaunchKernelGGL(k_flag_clear, dim3(1), dim3(64), 0, st, flag_dev);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || count == 0) return e;
  int64_t blocks = ((count >> 2) + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;  // 16 workgroups per CU, then a grid-stride loop
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_check_finite, dim3((unsigned)blocks), dim3(256), 0, st, W, count, flag_dev);
  return hipGetLastError();
}

hipError_t launch_topk(const double* e, int n, int k, int* idx, hipStream_t st) {
  if (k == 0 || n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk, dim3(1), dim3(1024), 0, st, e, n, k, idx);
  return hipGetLastError();
}

}  // namespace nf4k
