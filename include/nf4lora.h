/*
 * libnf4lora: the QLoRA linear layer on an NF4-quantized frozen base, for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The layer is equation (3) of "QLoRA: How to fine-tune large language
 * models with less memory" ("The algebra" section):
 *     Y = X W + s X L1 L2
 * with the frozen W stored 4-bit NF4 ("1. NormalFloat"), one scale per block
 * of 64 weights, optionally double quantized ("2. Double quantization").
 * Only the adapters L1, L2 and the input X receive gradients; the frozen W
 * is read, never differentiated ("Lesson 17. What QLoRA Actually Costs",
 * Warm-up).
 *
 * Conventions used by every entry point
 * -------------------------------------
 * - W is stored [rows][cols] row-major: rows = o (outputs), cols = h
 *   (inputs), the usual layout of a linear layer's weight; X W in the
 *   equation is X * W_st^T here.
 * - bf16 values travel as uint16_t bit patterns.  X [M][h], dY [M][o],
 *   Y [M][o], dX [M][h], T [M][r] are row-major bf16; L1 [h][r] and
 *   L2 [r][o] are row-major bf16; dL1 [h][r] and dL2 [r][o] are fp32.
 * - Every pointer argument except the nf4_tensor descriptor itself and the
 *   host scalars is a DEVICE pointer, and every device base pointer must be
 *   16-byte aligned (NF4_ERR_ALIGN otherwise).
 * - The caller owns every buffer.  The library allocates and frees nothing,
 *   keeps no mutable global state, and is safe to call from several host
 *   threads (calls on one stream run in stream order).
 * - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *   asynchronously; nothing synchronizes.  Arguments are validated before
 *   any launch and the first failure is returned; a failed launch returns
 *   NF4_ERR_HIP; faults inside kernels surface at the caller's next
 *   synchronization.  No C++ exception crosses this boundary.
 * - Outputs must not overlap inputs (NF4_ERR_ALIAS).
 * - Results are deterministic: all reductions run in a fixed order (no
 *   floating-point atomics), so repeated calls give identical bits.
 */
#ifndef NF4LORA_H
#define NF4LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NF4LORA_ABI_VERSION 5

/*
 * Status codes.  Values 0..7 are fixed since the first release of this ABI;
 * NF4_ERR_NONFINITE was appended later, so it follows NF4_ERR_ARG.
 */
typedef enum nf4_status {
  NF4_OK = 0,
  NF4_ERR_NULL = 1,       /* a required pointer is NULL */
  NF4_ERR_SHAPE = 2,      /* a size is out of range or the sizes disagree */
  NF4_ERR_ALIGN = 3,      /* a device pointer is not 16-byte aligned */
  NF4_ERR_WORKSPACE = 4,  /* workspace NULL or smaller than nf4_workspace_bytes() */
  NF4_ERR_ALIAS = 5,      /* an output buffer overlaps an input buffer */
  NF4_ERR_HIP = 6,        /* a HIP runtime call or kernel launch failed */
  NF4_ERR_ARG = 7,        /* unsupported option (block size, group size, op id) */
  NF4_ERR_NONFINITE = 8   /* nf4_check_finite found an infinity or a NaN */
} nf4_status;

/*
 * Quantized weight descriptor (host struct; the buffers it points to are
 * device memory owned by the caller).
 *   rows, cols : W is [rows][cols]; cols % block == 0; rows >= 0.
 *   block      : weights per scale block along a row; must be 64 (the block
 *                size of "1. NormalFloat" / AQLoRA section 3.1).
 *   dq_group   : 0  -> absmax is float[nblocks] (fp32 per block);
 *                256 -> absmax is uint8[nblocks] (8-bit scale codes) and
 *                dq_scale is float[ceil(nblocks/256)], one fp32 step per
 *                group of 256 blocks ("2. Double quantization").
 *   codes      : rows*cols/2 bytes; byte t holds element 2t in its low
 *                nibble and element 2t+1 in its high nibble (row-major order).
 *   codebook   : the 16 code values (NF4_CODEBOOK_*, see nf4_codebook_values):
 *                NF4 (the format of "1. NormalFloat"), or, for comparison
 *                at identical storage, the symmetric int4 grid (c-8)/7
 *                ("Lesson 17. What QLoRA Actually Costs": int4 rather than
 *                NF4) or the E2M1 4-bit float / 6 (the ordinary-float curve of
 *                the QLoRA blog's figure 3).  Zero-initialised descriptors
 *                are NF4.
 *   residual   : NULL, or a second tensor of the same rows, cols, block,
 *                dq_group and codebook (with no residual of its own) that
 *                holds the quantized residual of this one: the second NF4
 *                stage of AQLoRA's additional controls (section 7).
 *                nf4_quantize then fills both (second stage: quantize
 *                fl32(w - w_hat1)), and every consumer uses
 *                w_hat = fl32(w_hat1 + w_hat2).
 * Dequantized weight: w_hat = fl32(table[code] * scale), scale = absmax
 * (fp32) or fl32(c8 * dq_scale[group]).  nblocks = rows*cols/64.
 */
typedef struct nf4_tensor {
  int64_t rows;
  int64_t cols;
  int32_t block;
  int32_t dq_group;
  uint8_t *codes;
  void *absmax;
  float *dq_scale;
  int32_t codebook;
  const struct nf4_tensor *residual;
} nf4_tensor;

/* Codebooks for nf4_tensor.codebook and nf4_layer_error. */
enum { NF4_CODEBOOK_NF4 = 0, NF4_CODEBOOK_INT4 = 1, NF4_CODEBOOK_FP4 = 2 };

/* Operation ids for nf4_workspace_bytes. */
enum { NF4_OP_FWD = 1, NF4_OP_BWD = 2, NF4_OP_ERROR = 3, NF4_OP_CHECK = 4 };

/* ABI version of the loaded library (NF4LORA_ABI_VERSION). */
int nf4_abi_version(void);

/* Static string naming a status code; never NULL. */
const char *nf4_status_str(int status);

/*
 * The 16 NF4 code values (fp32, ascending) the kernels use, written to the
 * HOST array out[16].  They are normal quantiles at evenly spaced
 * probabilities, seven negative, an exact zero and eight positive, each side
 * scaled so its outermost value is exactly -1 or +1 (the NormalFloat layout
 * of "1. NormalFloat", QLoRA blog).  Computed once in fp64 by the library's
 * own inverse normal CDF and rounded to nearest fp32.
 */
void nf4_code_table(float out[16]);

/*
 * The 16 code values of a codebook (fp32, ascending; equal values keep their
 * order), written to the HOST array out[16]:
 *   NF4_CODEBOOK_NF4  : as nf4_code_table;
 *   NF4_CODEBOOK_INT4 : (c - 8) / 7, the fp64 quotient rounded to fp32;
 *   NF4_CODEBOOK_FP4  : -6 -4 -3 -2 -1.5 -1 -.5 -0 +0 .5 1 1.5 2 3 4 6, each / 6
 *                       (fp64 quotient rounded to fp32).
 * The encoder picks the nearest value to x = w / absmax, the lower code on a
 * tie (so fp4 never yields +0 and int4 never its code 0, -8/7).
 * Errors: NF4_ERR_NULL, _ARG (unknown codebook).
 */
nf4_status nf4_codebook_values(int32_t codebook, float out[16]);

/*
 * Byte sizes of the three buffers of a quantized [rows][cols] weight
 * (host outputs; any may be NULL).  Storage follows the worked 65B budget in
 * the QLoRA blog: 0.5 byte/weight of codes, plus 4 bytes per 64-weight block
 * without double quantization, or 1 byte per block + 4 bytes per 256 blocks
 * with it.  Errors: NF4_ERR_SHAPE, NF4_ERR_ARG.
 */
nf4_status nf4_tensor_bytes(int64_t rows, int64_t cols, int32_t block, int32_t dq_group,
                            size_t *codes_bytes, size_t *absmax_bytes, size_t *dq_scale_bytes);

/*
 * Non-finite input.  The pages define the format for real-valued weights
 * only; every pass over an fp32 W (nf4_quantize, nf4_quantize_error,
 * nf4_layer_error, nf4_layer_error_batch, nf4lora_merge) takes finite values
 * as a precondition and does not check it: an Inf or NaN weight gives
 * unspecified codes and scales for its block and a NaN error for its layer
 * (nf4_topk ranks NaN errors first).  The checked mode is this call, made
 * before the pass:
 *
 * nf4_check_finite scans W (device fp32, `count` values) and returns NF4_OK
 * when every value is finite, NF4_ERR_NONFINITE when any is an infinity or a
 * NaN.  Unlike every other entry point it SYNCHRONIZES `stream` (it reads its
 * answer back to the host), so it cannot be captured into a graph.
 *   ws: nf4_workspace_bytes(NF4_OP_CHECK, ...) bytes (256), 16-byte aligned,
 *       not overlapping W.
 * count == 0 returns NF4_OK without a launch.  Errors: NF4_ERR_NULL, _SHAPE
 * (count < 0), _ALIGN, _ALIAS, _WORKSPACE, _HIP, _NONFINITE.
 */
nf4_status nf4_check_finite(const float *W, int64_t count, void *ws, size_t ws_bytes, void *stream);

/*
 * Blockwise NF4 quantization of W (device fp32 [rows][cols], finite values)
 * into the buffers of *q ("1. NormalFloat" and "2. Double quantization",
 * QLoRA blog):
 *   a_b  = max |w| over each block of 64;
 *   x    = w / a_b (IEEE fp32 division; 0 for an all-zero block);
 *   code = the nearest table value to x, the lower code on an exact tie;
 *   with dq_group = 256, per group: S = fl32(max a_b / 255),
 *   c8 = min(255, round-half-even(fl32(a_b / S))) (0 when S = 0).
 * Codes do not depend on dq_group.  rows * cols is at most
 * (2^24 - 1) * 2^14 (about 2.7e11 weights: one launch of 256-thread
 * workgroups, one per 16384 weights, stays below 2^32 work-items; the same
 * bound applies to nf4_quantize_error, nf4_layer_error and each linear of
 * nf4_layer_error_batch).  Errors: NF4_ERR_NULL, _SHAPE, _ARG, _ALIGN,
 * _ALIAS, _HIP.
 */
nf4_status nf4_quantize(const float *W, const nf4_tensor *q, void *stream);

/*
 * Dequantize *q into W_out [rows][cols]: fp32 w_hat when out_is_bf16 == 0,
 * else the bf16 round-to-nearest-even of w_hat ("1. NormalFloat": weights
 * are reconstructed into bf16 before the matmul).  Errors as nf4_quantize.
 */
nf4_status nf4_dequantize(const nf4_tensor *q, void *W_out, int32_t out_is_bf16, void *stream);

/*
 * Workspace bytes for an operation (host output *bytes).
 *   op = NF4_OP_FWD or NF4_OP_BWD: M tokens, W [rows][cols], rank r;
 *   op = NF4_OP_ERROR: W [rows][cols] (M and r ignored);
 *   op = NF4_OP_CHECK: nf4_check_finite (all sizes ignored).
 * Errors: NF4_ERR_NULL, _SHAPE, _ARG.
 */
nf4_status nf4_workspace_bytes(int32_t op, int64_t M, int64_t rows, int64_t cols, int32_t r,
                               size_t *bytes);

/*
 * Forward pass, equation (3): T = X L1 and Y = X W_hat^T + s T L2 with the
 * NF4 weight dequantized to bf16 inside the matmul (never written out) and
 * fp32 accumulation.  s is alpha/r ("LoRA: Fine-tuning a model by learning a
 * small update", the algebra section; rsLoRA callers pass alpha/sqrt(r)).
 *   W    : quantized [o][h], h % 64 == 0, o % 64 == 0, h and o at most
 *          4194304 and o * h at most 2^32 (the fused kernels address a
 *          256-row activation tile and the packed codes through 32-bit buffer
 *          ranges); larger weights are rejected with NF4_ERR_SHAPE.
 *   X    : bf16 [M][h]; M >= 0 (M == 0 does nothing).
 *   L1   : bf16 [h][r];  L2 : bf16 [r][o];  1 <= r <= 256.
 *   Y    : bf16 [M][o] output.
 *   T_out: bf16 [M][r] output (X L1, to hand to nf4lora_bwd), or NULL.
 *   ws   : device workspace of at least nf4_workspace_bytes(NF4_OP_FWD,...).
 * Errors: NF4_ERR_NULL, _SHAPE, _ARG, _ALIGN, _WORKSPACE, _ALIAS, _HIP.
 */
nf4_status nf4lora_fwd(const nf4_tensor *W, const uint16_t *X, int64_t M,
                       const uint16_t *L1, const uint16_t *L2, int32_t r, float s,
                       uint16_t *Y, uint16_t *T_out,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * nf4lora_fwd for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results (bit for bit) and errors as nf4lora_fwd, without the
 * workspace: the library uses a fixed device area of 16 MiB per GPU instead,
 * created with the library's code object on each GPU it runs on and held
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).
 *   - A layer whose forward workspace (nf4_workspace_bytes(NF4_OP_FWD, ...))
 *     exceeds 16 MiB is rejected with NF4_ERR_WORKSPACE before any HIP call
 *     (layers from 4096 x 4096 at 2048 tokens to 28672 x 8192 at 16384
 *     tokens need 0.07 to 14.5 MiB at r <= 64; r = 256 at M = 16384 and
 *     o = 28672 needs 58 MiB: use nf4lora_fwd there).
 *   - Every call on a GPU shares that GPU's area, and the area keeps the last
 *     call's contents; each call clears what must start at zero with a kernel
 *     of its own (no memset).  Calls that overlap on one GPU (several streams
 *     or host threads at once) race on the area: serialize them.
 *   - The first call on a device looks up the area's device address
 *     (hipGetSymbolAddress) with that device current; later calls reuse it.
 */
nf4_status nf4lora_fwd_noalloc(const nf4_tensor *W, const uint16_t *X, int64_t M,
                               const uint16_t *L1, const uint16_t *L2, int32_t r, float s,
                               uint16_t *Y, uint16_t *T_out, void *stream);

/*
 * Backward pass of equation (3) for the adapters and the input; the frozen
 * W gets no gradient ("Lesson 17", Warm-up):
 *   G   = s dY L2^T                 (bf16 [M][r], internal)
 *   dL2 = s T^T dY                  -> fp32 [r][o]
 *   dL1 = X^T G                     -> fp32 [h][r]
 *   dX  = dY W_hat + G L1^T         -> bf16 [M][h], optional
 *   T   : the forward's T_out (bf16 [M][r]), or NULL to recompute X L1.
 *   dX  : NULL skips the input gradient (the early backward stop of
 *         AQLoRA's speed setting, section 3.3 Adapter placement).
 * M == 0 writes zeros to dL1 and dL2.  Shapes and errors as nf4lora_fwd.
 */
nf4_status nf4lora_bwd(const nf4_tensor *W, const uint16_t *X, const uint16_t *dY, int64_t M,
                       const uint16_t *L1, const uint16_t *L2, int32_t r, float s,
                       const uint16_t *T, uint16_t *dX, float *dL1, float *dL2,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * The same layer with the frozen weight kept in bf16 instead of NF4: the
 * protected linears of AQLoRA (section 3.2 Precision allocation: the K
 * linears with the largest NF4 reconstruction error stay in 16-bit and skip
 * the per-step dequantization).  W is bf16 [rows = o][cols = h] with rows and
 * cols multiples of 64 and rows * cols < 2^31; it feeds the same fused
 * kernels (no dequantization step).  Every other argument, the workspace
 * (nf4_workspace_bytes with the same rows and cols), the outputs and the
 * errors are those of nf4lora_fwd / nf4lora_bwd.
 */
nf4_status bf16lora_fwd(const uint16_t *W, int64_t rows, int64_t cols, const uint16_t *X, int64_t M,
                        const uint16_t *L1, const uint16_t *L2, int32_t r, float s,
                        uint16_t *Y, uint16_t *T_out,
                        void *ws, size_t ws_bytes, void *stream);
nf4_status bf16lora_bwd(const uint16_t *W, int64_t rows, int64_t cols, const uint16_t *X,
                        const uint16_t *dY, int64_t M,
                        const uint16_t *L1, const uint16_t *L2, int32_t r, float s,
                        const uint16_t *T, uint16_t *dX, float *dL1, float *dL2,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * Merge a trained adapter into the base ("LoRA: Fine-tuning a model by
 * learning a small update", section "Serving models and switching tasks":
 * W_merged = W0 + (alpha/r) B A; "Lesson 17. What QLoRA Actually Costs":
 * merge into the full-precision base, quantise afterwards if needed).  In
 * the storage layout [rows = o][cols = h]:
 *     W_out[n][k] = base[n][k] + s * sum_j L2[j][n] * L1[k][j]
 * computed in fp32 (fp32 sum of the r products, then s * sum + base).
 *   base : W (fp32 [rows][cols]) when W != NULL, else q dequantized exactly
 *          as nf4_dequantize does (q->rows, q->cols must equal rows, cols).
 *   L1   : bf16 [cols][r];  L2 : bf16 [r][rows];  1 <= r <= 256; both
 *          16-byte aligned.
 *   W_out: fp32 [rows][cols] (out_is_bf16 == 0) or its bf16 rounding to
 *          nearest even; for an NF4 re-quantization pass the fp32 form to
 *          nf4_quantize.
 * rows >= 0, cols % 64 == 0.  Errors: NF4_ERR_NULL, _SHAPE, _ARG, _ALIGN,
 * _ALIAS, _HIP.
 */
nf4_status nf4lora_merge(const float *W, const nf4_tensor *q, int64_t rows, int64_t cols,
                         const uint16_t *L1, const uint16_t *L2, int32_t r, float s,
                         void *W_out, int32_t out_is_bf16, void *stream);

/*
 * One linear of a stack run by nf4_stack_fwd / nf4_stack_bwd.  The frozen
 * weight is either NF4 (q) or a protected bf16 weight (w_bf16, [rows][cols]);
 * exactly one of the two is set.  r > 0 gives the linear an adapter (L1, L2,
 * s as in nf4lora_fwd); r == 0 means no adapter (AQLoRA's adapter placement,
 * section 3.3, leaves some linears without one): the forward is Y = X W^T
 * and the backward only carries dX.
 *   X  [M][h], Y [M][o], T [M][r] (saved by the forward when non-NULL and
 *   handed to the backward), dY [M][o], dX [M][h] or NULL, dL1 [h][r],
 *   dL2 [r][o].  All device pointers, caller-owned.
 */
typedef struct {
    const nf4_tensor *q;
    const uint16_t *w_bf16;
    int64_t rows, cols;
    int32_t r;
    float s;
    const uint16_t *L1, *L2;
    const uint16_t *X;
    uint16_t *Y, *T;
    const uint16_t *dY;
    uint16_t *dX;
    float *dL1, *dL2;
} nf4_linear;

/* Workspace bytes for running any linear of the stack (host output). */
nf4_status nf4_stack_workspace_bytes(const nf4_linear *layers, int32_t n, int64_t M, size_t *bytes);

/*
 * Forward over layers[0 .. n) in order, each as nf4lora_fwd / bf16lora_fwd
 * (or the plain product when r == 0), sharing one workspace.  Stops at the
 * first failing linear and returns its status.
 */
nf4_status nf4_stack_fwd(const nf4_linear *layers, int32_t n, int64_t M, void *ws, size_t ws_bytes,
                         void *stream);

/*
 * Backward over layers[n-1] down to layers[cut] (0 <= cut <= n): the early
 * backward stop of AQLoRA's speed setting (section 3.3 Adapter placement and
 * section 6: no computation below the cutoff).  Linears below cut are not
 * touched; a linear whose dX is NULL gets no input gradient (the lowest
 * adapted linears need none).  Each linear runs as nf4lora_bwd /
 * bf16lora_bwd, or as the plain input-gradient product when r == 0.
 */
nf4_status nf4_stack_bwd(const nf4_linear *layers, int32_t n, int32_t cut, int64_t M, void *ws,
                         size_t ws_bytes, void *stream);

/*
 * The fused NF4 matmul on its own (the base product inside nf4lora_fwd and
 * nf4lora_bwd), with an optional low-rank term in the same output tile:
 *   transpose = 0:  C [M][o] = A [M][h] * W_hat^T + A2 [M][R] * B2 [o][R]^T
 *   transpose = 1:  C [M][h] = A [M][o] * W_hat   + A2 [M][R] * B2 [h][R]^T
 * W_hat is dequantized to bf16 inside the kernel (equation (3) base term of
 * the QLoRA blog, "1. NormalFloat": bf16 reconstruction before the matmul);
 * fp32 accumulation, bf16 C.  R is a multiple of 16 in [0, 256] (pad the
 * low-rank operands with zero columns); A2 and B2 may be NULL only when
 * R == 0.  Shapes as nf4lora_fwd (W rows and cols multiples of 64).
 * Errors: NF4_ERR_NULL, _SHAPE, _ARG, _ALIGN, _ALIAS, _HIP.
 */
nf4_status nf4_matmul(const nf4_tensor *W, int32_t transpose, const uint16_t *A, int64_t M,
                      const uint16_t *A2, const uint16_t *B2, int32_t R, uint16_t *C, void *stream);

/*
 * Per-layer NF4 reconstruction error of W (device fp32 [rows][cols]):
 *   e = sqrt(sum (w - w_hat)^2) / sqrt(sum w^2)   (0 when W is all zero),
 * w_hat from 64-weight blocks (dq_group 0) or with double quantization
 * (dq_group 256).  This is the ranking quantity of AQLoRA's profiling pass
 * (section 3.1; the page's equation is missing, the relative Frobenius norm
 * is the reading).  codebook as in nf4_tensor (NF4 for the ranking; the
 * others measure the comparison at identical storage).  The decoded value is
 * fp32 as the format defines; the difference and the squares are fp64, each
 * square added with a fused multiply-add in a fixed order, and the per-group
 * sums are added in a fixed order.  err_dev: device double[1].  ws: nf4_workspace_bytes(NF4_OP_ERROR).
 * Errors: NF4_ERR_NULL, _SHAPE, _ARG, _ALIGN, _WORKSPACE, _HIP.
 */
nf4_status nf4_layer_error(const float *W, int64_t rows, int64_t cols, int32_t block,
                           int32_t dq_group, int32_t codebook, double *err_dev, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * nf4_quantize and nf4_layer_error from one read of W: quantizes W into *q
 * exactly as nf4_quantize does, and writes to err_dev the value that
 * nf4_layer_error(W, q->rows, q->cols, 64, err_dq_group, q->codebook, ...)
 * returns, bit for bit (AQLoRA section 3.1 ranks the layers by this error;
 * the QLoRA blog's "1. NormalFloat" and "2. Double quantization" define the
 * codes and scales).  One stage only: q->residual must be NULL.
 *   err_dq_group: 0 (error with the plain block absmax as scale) or
 *                 q->dq_group (with the double-quantized scales).
 *   ws:           nf4_workspace_bytes(NF4_OP_ERROR, ...) bytes, 16-byte aligned.
 * W, the buffers of *q, ws and err_dev must not overlap.
 * Errors: NF4_ERR_NULL, _SHAPE, _ARG (residual set, err_dq_group not 0 or
 * q->dq_group), _ALIGN, _ALIAS, _WORKSPACE, _HIP.
 */
nf4_status nf4_quantize_error(const float *W, const nf4_tensor *q, int32_t err_dq_group, double *err_dev,
                              void *ws, size_t ws_bytes, void *stream);

/*
 * The profiling pass over a whole model at once: AQLoRA section 3.1 measures
 * the NF4 reconstruction error of every linear before it ranks them.  For
 * i < n, err_dev[i] is bit for bit what nf4_layer_error(W[i], rows[i],
 * cols[i], 64, dq_group, codebook, ...) writes.  Up to 64 linears go into one
 * launch pair, so n linears cost about 2 n / 64 launches instead of 2 n.
 *   W:          host array of n device pointers, each fp32 [rows[i]][cols[i]],
 *               16-byte aligned (NULL allowed only for an empty linear).
 *   rows, cols: host arrays of n shapes; cols[i] % 64 == 0.
 *   err_dev:    device double[n], 8-byte aligned.
 *   ws:         nf4_error_batch_workspace_bytes(rows, cols, n) bytes, 16-byte
 *               aligned: one 16-byte partial per group of 256 blocks of every
 *               linear.
 * The host arrays are read during the call only.  n == 0 does nothing.  ws
 * and err_dev must not overlap each other or any W[i].
 * Errors: NF4_ERR_NULL, _SHAPE, _ARG (n < 0, dq_group, codebook), _ALIGN,
 * _ALIAS, _WORKSPACE, _HIP.
 */
nf4_status nf4_layer_error_batch(const float *const *W, const int64_t *rows, const int64_t *cols, int32_t n,
                                 int32_t dq_group, int32_t codebook, double *err_dev, void *ws, size_t ws_bytes,
                                 void *stream);
/* Workspace bytes of nf4_layer_error_batch over these shapes (host output *bytes).
 * Errors: NF4_ERR_NULL, _SHAPE, _ARG (n < 0). */
nf4_status nf4_error_batch_workspace_bytes(const int64_t *rows, const int64_t *cols, int32_t n, size_t *bytes);

/*
 * The protected set of AQLoRA's precision allocation (section 3.2): indices
 * of the k largest of n errors (device double[n]), largest first, equal
 * errors ordered by lower index, written to device int32 idx_dev[k].  A NaN
 * error (the layer of a non-finite weight) ranks above every number, NaNs
 * among themselves by index, so the order is total and idx_dev is always a
 * set of k distinct indices.
 * 0 <= k <= n <= 65536.  Errors: NF4_ERR_NULL, _SHAPE, _ALIGN, _HIP.
 */
nf4_status nf4_topk(const double *err_dev, int32_t n, int32_t k, int32_t *idx_dev, void *stream);

/*
 * Protection count for a budget rho over n linears: round-half-up(rho * n)
 * (AQLoRA section 3.2; K = 29 at rho = .2 over 144 linears).  Host only;
 * returns -1 for rho outside [0, 1] or n < 0.
 */
int32_t nf4_protect_count(double rho, int32_t n);

/*
 * Measurement aid, not part of the layer: the bf16 matrix-core rate with no
 * memory or LDS traffic, the ceiling the fused GEMM's MFMA work is compared
 * with beside the dense peak.  Launches `workgroups` workgroups of 512
 * threads; every wave issues iters * 8 v_mfma_f32_32x32x16_bf16 (32768 flops
 * each: 2.62e5 * iters flops per wave; iters rounded up to an even count) on
 * eight independent accumulators with
 * pseudo-random bf16 operands, and writes one float per thread to out_dev
 * (device float[workgroups * 512]) so the work is kept.  Asynchronous.
 * Errors: NF4_ERR_NULL, _SHAPE (iters < 1, workgroups < 1 or > 2^20), _ALIGN,
 * _HIP.
 */
nf4_status nf4_probe_mfma_peak(int32_t iters, int32_t workgroups, float *out_dev, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NF4LORA_H */
