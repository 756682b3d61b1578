"""NF4 blockwise quantization, double quantization, dequantization, error.

Test infrastructure only (see the package docstring).

Layout: W is [rows][cols] fp32 row-major (rows = o outputs, cols = h inputs,
the weight of a linear layer), cols a multiple of the block size.  Flattened
element i belongs to block i // block; with cols % block == 0 no block crosses
a row.  Double-quant groups are consecutive runs of `dq_group` blocks (the
last group may be shorter).
"""
from __future__ import annotations

import math
import statistics
from dataclasses import dataclass

import numpy as np
import torch

BLOCK = 64


def nf4_table() -> np.ndarray:
    """The 16 NF4 code values, fp32, ascending.

    "QLoRA: How to fine-tune large language models with less memory", section
    "1. NormalFloat": 16 codes laid out for a zero-centred normal distribution,
    denser near zero.  The pages give no formula; the reading used here is the
    published NF4 construction: normal quantiles at evenly spaced
    probabilities between 1/2 and delta = 1 - (1/30 + 1/32)/2, eight on the
    positive side and seven on the negative side, each side divided by the
    outermost quantile so the ends are exactly -1 and +1, plus an exact zero.
    Computed in fp64, then rounded to nearest fp32.
    """
    inv = statistics.NormalDist().inv_cdf
    delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    z = inv(delta)
    pos = [inv(delta - j * (delta - 0.5) / 8.0) / z for j in range(8)]
    neg = [-inv(delta - j * (delta - 0.5) / 7.0) / z for j in range(7)]
    vals = sorted(pos + neg + [0.0])
    return np.array(vals, dtype=np.float64).astype(np.float32)


CODEBOOKS = ("nf4", "int4", "fp4")


def codebook_table(codebook: str = "nf4") -> np.ndarray:
    """The 16 code values of a 4-bit codebook, fp32, ascending (equal values keep their order).

    nf4   the NormalFloat table above.
    int4  the integer alternative ("Lesson 17. What QLoRA Actually Costs",
          the "int4 rather than NF4" row of its comparison table): the pages
          give no layout; the reading taken is the symmetric absmax int4 grid,
          code c -> (c - 8) / 7, so that -1, 0 and +1 are codes 1, 8 and 15
          (code 0, -8/7, lies outside [-1, 1] and is never chosen).
    fp4   the ordinary 4-bit float of the QLoRA blog's figure 3 ("the blue
          ordinary-float curve"): the reading taken is the E2M1 format (sign,
          2 exponent bits, 1 mantissa bit: magnitudes 0, .5, 1, 1.5, 2, 3, 4,
          6) divided by its largest value 6, with -0 before +0.  With the
          lower code on a tie, an exact zero and the small positive values
          nearest zero take -0; +0 is never chosen.
    Values that are not binary fractions are the fp64 quotient rounded to fp32.
    """
    if codebook == "nf4":
        return nf4_table()
    if codebook == "int4":
        return np.array([(c - 8) / 7.0 for c in range(16)], dtype=np.float64).astype(np.float32)
    if codebook == "fp4":
        mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
        neg = [-m / 6.0 for m in reversed(mags)]   # -1 .. -0
        pos = [m / 6.0 for m in mags]              # +0 .. +1
        neg[-1] = -0.0
        return np.array(neg + pos, dtype=np.float64).astype(np.float32)
    raise ValueError(f"unknown codebook {codebook!r}")


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: element 2t in the low nibble, 2t+1 in the high."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    assert c.size % 2 == 0
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0x0F
    out[1::2] = p >> 4
    return out


@dataclass
class NF4Quant:
    rows: int
    cols: int
    block: int
    dq_group: int
    codes: np.ndarray          # uint8 [rows*cols], one code per element (unpacked)
    absmax: np.ndarray         # fp32 [nblocks], first-level scale per block
    c8: np.ndarray | None      # uint8 [nblocks] when double quantized
    dq_scale: np.ndarray | None  # fp32 [ngroups] step per group when double quantized
    codebook: str = "nf4"

    @property
    def packed(self) -> np.ndarray:
        return pack_codes(self.codes)

    @property
    def nblocks(self) -> int:
        return self.rows * self.cols // self.block

    def scales(self) -> np.ndarray:
        """Scale applied at dequantization: fp32 absmax, or c8 * S_g (fp32)."""
        if self.dq_group == 0:
            return self.absmax
        g = np.arange(self.nblocks) // self.dq_group
        return (self.c8.astype(np.float32) * self.dq_scale[g]).astype(np.float32)


def _encode(x: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Nearest table entry by absolute difference; the first (lower) index wins ties.

    Differences are taken in fp64 from fp32 operands; near any decision point
    x and the two candidate codes are of similar size, so the comparison is
    exact there (the fp64 difference of two fp32 values within a factor of
    2^29 of each other is exact).
    """
    q = table.astype(np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 20
    for s in range(0, flat_x.size, step):
        d = np.abs(flat_x[s:s + step].astype(np.float64)[:, None] - q[None, :])
        flat_o[s:s + step] = np.argmin(d, axis=1)
    return out


def quantize(W, block: int = BLOCK, dq_group: int = 0, codebook: str = "nf4") -> NF4Quant:
    """Blockwise absmax NF4 quantization, optionally with double quantization.

    Steps ("1. NormalFloat" and "2. Double quantization" in the QLoRA blog):
      1. absmax a_b = max |w| over each block of `block` consecutive weights (fp32).
      2. x = w / a_b, IEEE fp32 division; x = 0 for an all-zero block.
      3. code = index of the nearest code value to x (lower index on a tie);
         the NF4 table unless another codebook is named.
      4. double quant (dq_group > 0), run after encoding so codes do not change:
         per group of dq_group blocks, S_g = fl32(max a / 255) and
         c8_b = min(255, round-half-even(fl32(a_b / S_g))), c8 = 0 if S_g = 0.
         The pages fix 8 bits per first-level scale and one wider scale per
         group of 256; the linear unsigned 8-bit map is the reading taken.
    """
    W = np.ascontiguousarray(np.asarray(W, dtype=np.float32))
    rows, cols = W.shape
    if cols % block != 0:
        raise ValueError("cols must be a multiple of the block size")
    blocks = W.reshape(-1, block)
    absmax = np.max(np.abs(blocks), axis=1).astype(np.float32)
    safe = np.where(absmax == 0, np.float32(1), absmax).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)          # fp32 / fp32: IEEE division
    x[absmax == 0, :] = np.float32(0)
    codes = _encode(x, codebook_table(codebook)).reshape(-1)
    c8 = S = None
    if dq_group:
        nb = absmax.size
        ng = (nb + dq_group - 1) // dq_group
        S = np.empty(ng, dtype=np.float32)
        for g in range(ng):
            m = absmax[g * dq_group:(g + 1) * dq_group].max()
            S[g] = np.float32(m) / np.float32(255)
        Sb = S[np.arange(nb) // dq_group]
        safeS = np.where(Sb == 0, np.float32(1), Sb).astype(np.float32)
        r = np.rint((absmax / safeS).astype(np.float32))
        c8 = np.minimum(np.float32(255), r).astype(np.uint8)
        c8[Sb == 0] = 0
    return NF4Quant(rows, cols, block, dq_group, codes, absmax, c8, S, codebook)


def dequantize(q: NF4Quant) -> np.ndarray:
    """w_hat = fl32(table[code] * scale_b), fp32 [rows][cols]."""
    t = codebook_table(q.codebook)
    sc = q.scales()
    w = t[q.codes].reshape(-1, q.block) * sc[:, None]
    return w.astype(np.float32).reshape(q.rows, q.cols)


def bf16_bits(w) -> np.ndarray:
    """bf16 round-to-nearest-even of fp32 values, as uint16 bit patterns.

    "QLoRA: How to fine-tune large language models with less memory", section
    "1. NormalFloat": the stored weights are reconstructed into bf16 for the
    matmul.  bf16 keeps the sign, the 8 exponent bits and the top 7 mantissa
    bits of fp32; the value is rounded to the nearer of the two neighbouring
    bf16 values, the one with an even last mantissa bit on an exact tie
    (IEEE round-to-nearest-even, the rounding the pages leave implicit).
    Subnormals are kept; values past the largest finite bf16 go to infinity.
    The library routine (torch's fp32 -> bfloat16 conversion) is one step.
    """
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(w, dtype=np.float32))).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def dequantize_bf16_bits(q: NF4Quant) -> np.ndarray:
    """The bf16 operand form of w_hat: bf16_bits of the fp32 dequantized weight."""
    return bf16_bits(dequantize(q))


def quantize_residual(W, block: int = BLOCK, dq_group: int = 0, codebook: str = "nf4"):
    """Two-stage quantization: the weight, then what the first stage missed.

    AQLoRA summary, section 7 (additional controls): a second NF4 stage over
    the residuals of the first also works.  The pages give no further detail;
    the reading taken is the plain one: q1 = quantize(W); the residual
    R = fl32(W - w_hat1) (fp32 subtraction of the first stage's dequantized
    weight); q2 = quantize(R) with the same block, double-quant group and
    codebook.  Returns (q1, q2).
    """
    W = np.ascontiguousarray(np.asarray(W, dtype=np.float32))
    q1 = quantize(W, block, dq_group, codebook)
    R = (W - dequantize(q1)).astype(np.float32)
    return q1, quantize(R, block, dq_group, codebook)


def dequantize_residual(q1: NF4Quant, q2: NF4Quant) -> np.ndarray:
    """The two-stage weight: w_hat = fl32(w_hat1 + w_hat2), fp32 [rows][cols]."""
    return (dequantize(q1) + dequantize(q2)).astype(np.float32)


def layer_error(W, block: int = BLOCK, dq_group: int = 0, codebook: str = "nf4") -> float:
    """Relative Frobenius NF4 reconstruction error ||W - W_hat||_F / ||W||_F, fp64.

    AQLoRA summary, section 3.1: each linear's weights are evaluated in
    64-element NF4 blocks and a per-layer reconstruction error is formed (the
    equation itself is missing from the page; the relative Frobenius norm is
    the reading taken).  0 for an all-zero W.
    """
    W = np.asarray(W, dtype=np.float32)
    wh = dequantize(quantize(W, block, dq_group, codebook))
    d = W.astype(np.float64) - wh.astype(np.float64)
    num = float(np.sum(d * d))
    den = float(np.sum(W.astype(np.float64) ** 2))
    if den == 0.0:
        return 0.0
    return math.sqrt(num) / math.sqrt(den)


def storage_bytes(rows: int, cols: int, block: int = BLOCK, dq_group: int = 0):
    """(codes, first-level scales, second-level scales) in bytes.

    4-bit codes; fp32 absmax per block without double quant; with double
    quant one byte per block plus one fp32 per group of dq_group blocks
    ("2. Double quantization" and the 65B worked budget in the QLoRA blog).
    """
    n = rows * cols
    nb = n // block
    codes = n // 2
    if dq_group == 0:
        return codes, 4 * nb, 0
    ng = (nb + dq_group - 1) // dq_group
    return codes, nb, 4 * ng


def protect_count(rho: float, n_layers: int) -> int:
    """Number of protected layers for a budget rho over n linears: round half up of rho*n.

    AQLoRA summary, section 3.2 (K fixed by the protection budget) and
    section 7 (K = 29 at rho = .2 on phi-1.5's 144 linears).
    """
    return int(math.floor(rho * n_layers + 0.5))


def topk(errors, k: int) -> list[int]:
    """Indices of the k largest errors, largest first; equal errors -> lower index first.

    AQLoRA summary, section 3.2: a fixed top-K cut keeps the highest-error
    layers at high precision.  The pages assume finite weights; an error that
    is NaN (a weight with an Inf or NaN in it) ranks above every number, and
    NaNs among themselves by index (the reading taken: the layer that cannot
    be measured is the first one kept out of 4-bit storage).
    """
    e = [float(v) for v in errors]
    order = sorted(range(len(e)), key=lambda i: (0, 0.0, i) if math.isnan(e[i]) else (1, -e[i], i))
    return order[:k]
