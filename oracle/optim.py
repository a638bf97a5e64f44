"""Adapter optimizer step (AdamW) in float64.  TEST INFRASTRUCTURE ONLY.

The pages place the optimizer after the backward pass: only the adapters are
updated, the frozen base never is ([TT] §4 "One QLoRA Training Step, End to
End"; [MC] "One training step, from input to update"), and the optimizer
state may live in CPU memory and move to the GPU when needed ([TT] §7 "Paged
Optimizers"; [MC] "3. Paged optimizers"; [GO] "Idea three").  The pages do
not write the optimizer out.  Reading: AdamW with decoupled weight decay
(Loshchilov and Hutter, "Decoupled Weight Decay Regularization") in its usual
form:

    p <- p * (1 - lr * wd)
    m <- beta1 * m + (1 - beta1) * g
    v <- beta2 * v + (1 - beta2) * g^2
    p <- p - lr / (1 - beta1^t) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)

with t the 1-based step count.  Parameters are float32 master copies of L1 and
L2; g is dL1 / dL2 (float32).
"""
from __future__ import annotations

import numpy as np


def adamw_step(p, g, m, v, t: int, lr: float, beta1: float, beta2: float, eps: float, wd: float):
    """One AdamW step in float64.  Returns (p, m, v) as new float64 arrays."""
    if t < 1:
        raise ValueError("step count starts at 1")
    p = np.asarray(p, dtype=np.float64) * (1.0 - lr * wd)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    bc1 = 1.0 - beta1 ** t
    bc2 = 1.0 - beta2 ** t
    denom = np.sqrt(v) / np.sqrt(bc2) + eps
    p = p - (lr / bc1) * m / denom
    return p, m, v
