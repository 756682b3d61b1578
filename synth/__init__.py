"""Seeded synthetic inputs for the NF4-LoRA linear layer.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no quantization, no matmul, no error), so the CPU oracle
and the HIP path can both take their inputs from here without sharing any of
the computation they are compared on.

Workloads (W is stored [o][h] row-major, the frozen weight of a linear layer
mapping h inputs to o outputs; X is [M][h]; L1 is [h][r]; L2 is [r][o]; dY is
[M][o]).  The shapes are the Llama-style layers the workload table names:

  c1  512x512, r=8, M=128, NF4 blocks of 64, no double quant (CPU-scale case)
  c2  4096x4096 (a Llama-7B attention projection), r=16, M=2048, double quant
  c3  Llama-7B MLP trio: gate/up 4096->11008, down 11008->4096, r=64, M=8192,
      with 0.1% of weights turned into outliers x20
  c4  a 14B-shaped stack of 40 layers x 7 linears, per-linear sigma and tail
      weight (Student-t), used for the per-layer error ranking
  c5  70B-shaped MLP up-projection 8192->28672, r=64, M=16384

Recipe: numpy PCG64 seeded with the workload number (c1 uses seed 0); draws
in the order W, X, L1, L2, dY; every normal is drawn in fp32; bf16 tensors are
fp32 draws rounded to nearest-even bf16 (torch's conversion).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Layer:
    """One linear layer workload: W [rows=o][cols=h], X [M][h], rank r."""
    name: str
    rows: int          # o, output width
    cols: int          # h, input width (multiple of 64)
    M: int             # tokens
    r: int
    s: float
    sigma: float
    dq_group: int      # 0 = fp32 absmax per block, 256 = double quant
    seed: int
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0


C1 = Layer("c1-512x512-r8", 512, 512, 128, 8, 2.0, 0.02, 0, 0)
C2 = Layer("c2-llama7b-attn-4096x4096-r16", 4096, 4096, 2048, 16, 2.0, 0.02, 256, 2)
C3_GATE = Layer("c3-llama7b-gate-4096to11008-r64", 11008, 4096, 8192, 64, 2.0, 0.02, 256, 3,
                outlier_frac=1e-3, outlier_mult=20.0)
C3_UP = Layer("c3-llama7b-up-4096to11008-r64", 11008, 4096, 8192, 64, 2.0, 0.02, 256, 30,
              outlier_frac=1e-3, outlier_mult=20.0)
C3_DOWN = Layer("c3-llama7b-down-11008to4096-r64", 4096, 11008, 8192, 64, 2.0, 0.02, 256, 31,
                outlier_frac=1e-3, outlier_mult=20.0)
C5 = Layer("c5-70b-up-8192to28672-r64", 28672, 8192, 16384, 64, 2.0, 0.015, 256, 5)

LAYERS = {l.name: l for l in (C1, C2, C3_GATE, C3_UP, C3_DOWN, C5)}


def bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 numpy array -> torch bf16 tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _hash_u24(i, j, seed: int):
    """Counter-based integer hash of (row i, column j, seed) to 24 bits, for int64
    numpy arrays or torch tensors alike: two multiply-xorshift rounds on 32 bits
    (every product stays below 2^60, so int64 never overflows)."""
    x = (i * 0x9E3779B1 + j * 0x85EBCA77 + seed * 0xC2B2AE3D) & 0xFFFFFFFF
    x = x ^ (x >> 16)
    x = (x * 0x045D9F3B) & 0xFFFFFFFF
    x = x ^ (x >> 16)
    x = (x * 0x045D9F3B) & 0xFFFFFFFF
    x = x ^ (x >> 16)
    return x >> 8


def hash_weight(rows, cols, seed: int) -> np.ndarray:
    """fp32 weights W[i][j] for the given row and column indices (numpy), uniform
    on [-2^-5, 2^-5) in steps of 2^-28: the 24-bit hash minus 2^23, times 2^-28,
    both exact in fp32.  Any block of a large weight can be drawn on its own."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    u = _hash_u24(i, j, seed)
    return (u - (1 << 23)).astype(np.float32) * np.float32(2.0 ** -28)


def hash_weight_rows_torch(row0: int, nrows: int, cols: int, seed: int, device) -> torch.Tensor:
    """Rows row0 .. row0+nrows-1 of the same weights as hash_weight, on a torch device."""
    i = torch.arange(row0, row0 + nrows, dtype=torch.int64, device=device)[:, None]
    j = torch.arange(cols, dtype=torch.int64, device=device)[None, :]
    u = _hash_u24(i, j, seed)
    return (u - (1 << 23)).to(torch.float32) * (2.0 ** -28)


def _normal(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def layer_weight(layer: Layer, rng: np.random.Generator | None = None) -> np.ndarray:
    rng = rng if rng is not None else np.random.default_rng(layer.seed)
    W = _normal(rng, (layer.rows, layer.cols), layer.sigma)
    if layer.outlier_frac > 0:
        n = W.size
        k = int(round(layer.outlier_frac * n))
        idx = rng.choice(n, size=k, replace=False)
        flat = W.reshape(-1)
        flat[idx] *= np.float32(layer.outlier_mult)
    return W


def layer_inputs(layer: Layer, M: int | None = None):
    """All inputs of one layer workload, drawn in the fixed order W, X, L1, L2, dY.

    Returns a dict: W fp32 numpy [o][h]; X, L1, L2, dY bf16 torch tensors (CPU).
    """
    M = layer.M if M is None else M
    rng = np.random.default_rng(layer.seed)
    W = layer_weight(layer, rng)
    X = bf16(_normal(rng, (M, layer.cols), 1.0))
    L1 = bf16(_normal(rng, (layer.cols, layer.r), 0.02))
    L2 = bf16(_normal(rng, (layer.r, layer.rows), 0.02))
    dY = bf16(_normal(rng, (M, layer.rows), 1.0))
    return dict(W=W, X=X, L1=L1, L2=L2, dY=dY, s=layer.s, r=layer.r, dq_group=layer.dq_group)


def random_case(seed: int, rows: int, cols: int, M: int, r: int, sigma: float = 0.02):
    """Small ad-hoc case (ragged shapes for edge tests). Same draw order as layer_inputs."""
    rng = np.random.default_rng(seed)
    W = _normal(rng, (rows, cols), sigma)
    X = bf16(_normal(rng, (M, cols), 1.0))
    L1 = bf16(_normal(rng, (cols, r), 0.02))
    L2 = bf16(_normal(rng, (r, rows), 0.02))
    dY = bf16(_normal(rng, (M, rows), 1.0))
    return dict(W=W, X=X, L1=L1, L2=L2, dY=dY)


# ---------------------------------------------------------------------------
# c4: a 14B-shaped stack (40 decoder layers x {q,k,v,o,gate,up,down})
# ---------------------------------------------------------------------------

C4_LAYERS = 40
C4_HIDDEN = 5120
C4_FFN = 13824
C4_LINEARS = (("q", C4_HIDDEN, C4_HIDDEN), ("k", C4_HIDDEN, C4_HIDDEN),
              ("v", C4_HIDDEN, C4_HIDDEN), ("o", C4_HIDDEN, C4_HIDDEN),
              ("gate", C4_FFN, C4_HIDDEN), ("up", C4_FFN, C4_HIDDEN),
              ("down", C4_HIDDEN, C4_FFN))  # (name, rows=o, cols=h)
C4_DFS = (3, 5, 30)
C4_TOPK = 8
C4_TOKENS = 4096
C4_SEED = 4


@dataclass(frozen=True)
class StackLinear:
    index: int
    layer: int
    kind: str
    rows: int
    cols: int
    sigma: float
    df: int
    seed: int


def c4_stack(n_layers: int = C4_LAYERS) -> list[StackLinear]:
    """Per-linear parameters: sigma ~ U(0.01, 0.04), df uniform over {3, 5, 30}."""
    rng = np.random.default_rng(C4_SEED)
    out = []
    i = 0
    for l in range(n_layers):
        for kind, rows, cols in C4_LINEARS:
            sigma = float(rng.uniform(0.01, 0.04))
            df = int(C4_DFS[int(rng.integers(0, len(C4_DFS)))])
            out.append(StackLinear(i, l, kind, rows, cols, sigma, df, 1000 + i))
            i += 1
    return out


def c4_weight(lin: StackLinear, device: str = "cpu") -> torch.Tensor:
    """W = sigma * sqrt((df-2)/df) * t_df, so that Var(W) = sigma^2.

    Drawn with torch's generator (seeded per linear) so that the full stack can
    be produced directly in device memory; the same call on 'cpu' is not the
    same stream, so a test that compares with the oracle copies the device
    tensor back rather than regenerating it.
    """
    g = torch.Generator(device=device)
    g.manual_seed(lin.seed)
    shape = (lin.rows, lin.cols)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    # chi-square(df) drawn as the sum of df squared standard normals, so every
    # draw goes through the one seeded generator.
    v = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(lin.df):
        u = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        v.addcmul_(u, u)
    t = z / torch.sqrt(v / lin.df)
    scale = lin.sigma * math.sqrt((lin.df - 2) / lin.df)
    return (t * scale).contiguous()
