"""The LoRA linear on a dequantized frozen base, forward and backward, fp64.

Test infrastructure only (see the package docstring).

Orientation: equation (3) of "QLoRA: How to fine-tune large language models
with less memory" ("The algebra" section) writes Y = X W + s X L1 L2 with W of
shape h x o.  Here the frozen weight is stored as its transpose, W_st [o][h]
(the layout of a linear layer's weight), so X W = X W_st^T.  Shapes: X [M][h],
L1 [h][r], L2 [r][o], Y and dY [M][o].

Inputs may be torch tensors (bf16 or fp32) or numpy arrays; bf16 values are
upcast exactly.  All products are formed in fp64 with numpy's matmul.
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def fwd(X, W_hat, L1, L2, s: float):
    """Forward pass, equation (3): T = X L1; Y = X W_hat_st^T + s T L2.

    Returns (Y [M][o], T [M][r]) in fp64.
    """
    X, W, A, B = _f64(X), _f64(W_hat), _f64(L1), _f64(L2)
    T = X @ A
    Y = X @ W.T + s * (T @ B)
    return Y, T


def adapter_grads(X, dY, L1, L2, s: float):
    """Adapter part of the backward pass of equation (3) (no dX).

    Chain rule on Y = X W_st^T + s (X L1) L2 for the two adapter factors:
        G   = s dY L2^T          [M][r]
        dL2 = s (X L1)^T dY      [r][o]
        dL1 = X^T G              [h][r]
    Every token contributes a separate term to dL1 and dL2, so the gradients
    of a batch are the sums of the gradients of any split of its tokens.
    Returns (G, dL1, dL2) in fp64.
    """
    X, dY, A, B = _f64(X), _f64(dY), _f64(L1), _f64(L2)
    T = X @ A
    G = s * (dY @ B.T)
    dL2 = s * (T.T @ dY)
    dL1 = X.T @ G
    return G, dL1, dL2


def bwd(X, dY, W_hat, L1, L2, s: float):
    """Backward pass of equation (3) for the adapters and the input.

    The frozen base gets no gradient: it is read at high precision to carry
    the gradient to X ("Lesson 17. What QLoRA Actually Costs", Warm-up; the
    QLoRA blog's "One training step" section).  With G, dL1, dL2 from
    adapter_grads:
        dX  = dY W_st + G L1^T   [M][h]
    Returns (dX, dL1, dL2, G) in fp64.
    """
    G, dL1, dL2 = adapter_grads(X, dY, L1, L2, s)
    dY, W, A = _f64(dY), _f64(W_hat), _f64(L1)
    dX = dY @ W + G @ A.T
    return dX, dL1, dL2, G


def merge(W_hat, L1, L2, s: float) -> np.ndarray:
    """Merged weight in storage layout [o][h]: W_hat_st + s (L1 L2)^T, fp64.

    "LoRA: Fine-tuning a model by learning a small update", section "Serving
    models and switching tasks": the scaled update is added to the base once.
    """
    W, A, B = _f64(W_hat), _f64(L1), _f64(L2)
    return W + s * (A @ B).T
