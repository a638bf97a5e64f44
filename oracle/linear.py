"""LoRA linear layer over a dequantized NF4 base weight, in float64.
TEST INFRASTRUCTURE ONLY (see package docstring).

[MC] "The algebra" (Eq. 3): Y = X W + s X L1 L2 with W of shape h x o, L1 of
shape h x r, L2 of shape r x o and a scalar s; [TT] §3: the frozen base term
uses the reconstructed weight and the adapter term adds a learned correction
scaled by alpha / r.  The base weight is frozen: [MC] Figure 1 and "One
training step" / [TT] §4 — gradients pass through the base computation into
the adapters and the base weight is never updated, so the backward returns dX,
dL1 and dL2 only (no dW).

The weight is passed as its float32 reconstruction in PyTorch's [o][h] order
(row n holds the n-th output's h input weights); X, L1, L2 and dY are given as
float arrays holding the exact values of their bf16 inputs.  Every product is
an exact-input float64 matmul; nothing is rounded to bf16 here.
"""
from __future__ import annotations

import numpy as np

from .nf4 import dequantize


def dequantized_weight(packed, qabsmax, scale2, mean, h: int, o: int) -> np.ndarray:
    """float32 [o][h] reconstruction of an NF4 + double-quantized weight."""
    return dequantize(packed, qabsmax, scale2, mean, h * o, out="f32").reshape(o, h)


def linear_fwd(w_oh: np.ndarray, x: np.ndarray, l1, l2, s: float):
    """Forward: returns (Y [M][o], T [M][r]) with T = X L1 and Y = X W + s T L2.

    r = 0 (l1 is None) means no adapter: Y = X W and T is None.
    """
    W = np.asarray(w_oh, dtype=np.float64).T            # h x o, the pages' orientation
    X = np.asarray(x, dtype=np.float64)
    Y = X @ W
    if l1 is None:
        return Y, None
    T = X @ np.asarray(l1, dtype=np.float64)
    Y = Y + float(s) * (T @ np.asarray(l2, dtype=np.float64))
    return Y, T


def linear_bwd(w_oh: np.ndarray, x: np.ndarray, dy: np.ndarray, l1, l2, s: float):
    """Backward of Y = X W + s X L1 L2 for an upstream gradient dY.

    With U = dY L2^T and T = X L1:
      dX  = dY W^T + s U L1^T
      dL1 = s X^T U
      dL2 = s T^T dY
    Returns (dX, dL1, dL2); dL1 and dL2 are None when r = 0.
    """
    W = np.asarray(w_oh, dtype=np.float64).T
    X = np.asarray(x, dtype=np.float64)
    dY = np.asarray(dy, dtype=np.float64)
    dX = dY @ W.T
    if l1 is None:
        return dX, None, None
    L1 = np.asarray(l1, dtype=np.float64)
    L2 = np.asarray(l2, dtype=np.float64)
    s = float(s)
    U = dY @ L2.T
    T = X @ L1
    dX = dX + s * (U @ L1.T)
    dL1 = s * (X.T @ U)
    dL2 = s * (T.T @ dY)
    return dX, dL1, dL2


def merged_weight(packed, qabsmax, scale2, mean, h: int, o: int, l1, l2, s: float) -> np.ndarray:
    """float32 [o][h] merge of the adapter into the base: W' = W_hat + s * L1 L2.

    [TT] §11 "Saving, Loading, and Merging QLoRA Adapters": the base is
    dequantized to a wider precision, the LoRA update added, and the result may
    be quantized again (adding another quantization error); [GO] "What it
    added up to" notes that trained adapters fit the quantized base.  In the
    pages' orientation W is h x o, so the stored [o][h] entry (n, k) gets
    s * sum_q L1[k][q] L2[q][n].  float32 steps: each product of two bf16
    values is exact in float32; the r products are summed in float32 in
    ascending q; then fp32(s * P) and fp32(W_hat + that).
    """
    wh = dequantized_weight(packed, qabsmax, scale2, mean, h, o)
    if l1 is None or np.asarray(l1).shape[1] == 0:
        return wh.copy()
    L1 = np.asarray(l1, dtype=np.float32)      # [h][r]
    L2 = np.asarray(l2, dtype=np.float32)      # [r][o]
    P = np.zeros((o, h), dtype=np.float32)
    for q in range(L1.shape[1]):
        P = P + np.outer(L2[q, :], L1[:, q]).astype(np.float32)
    return wh + np.float32(s) * P
