"""The elementwise glue between the NF4 linears of a transformer block, in float64.
TEST INFRASTRUCTURE ONLY (see package docstring).

[MC] "A closer look: Design choices and memory costs" ("Why does adapter
placement matter?"): a transformer block has attention layers and feed-forward
(FFN) layers, and QLoRA puts adapters on every linear layer of both.  The pages
name LLaMA 7B to 65B but do not spell out the FFN.  Reading: it is LLaMA's
gated feed-forward, whose two input projections G (gate) and U (up) meet in
H = SiLU(G) * U elementwise before the down projection, with
SiLU(g) = g * sigmoid(g) and sigmoid(g) = 1 / (1 + exp(-g)).  Its backward for
an upstream gradient dH is dU = dH * SiLU(G) and
dG = dH * U * SiLU'(G), SiLU'(g) = sigmoid(g) * (1 + g * (1 - sigmoid(g))).

Where several linears read the same input (q, k, v, gate and up all read the
block input), the input's gradient is the sum of their dX: grad_sum.

Inputs are float arrays holding the exact values of the bf16 tensors; nothing
is rounded here.
"""
from __future__ import annotations

import numpy as np


def sigmoid(g) -> np.ndarray:
    """1 / (1 + exp(-g)), written so that neither branch overflows."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu_gate_fwd(g, u) -> np.ndarray:
    """H = SiLU(G) * U."""
    g = np.asarray(g, dtype=np.float64)
    return g * sigmoid(g) * np.asarray(u, dtype=np.float64)


def silu_gate_bwd(g, u, dh):
    """(dG, dU) of H = SiLU(G) * U for the upstream gradient dH."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    sg = sigmoid(g)
    du = dh * (g * sg)
    dg = dh * u * (sg * (1.0 + g * (1.0 - sg)))
    return dg, du


def grad_sum(parts) -> np.ndarray:
    """Gradient of an input read by several linears: the sum of their input gradients."""
    out = np.zeros_like(np.asarray(parts[0], dtype=np.float64))
    for p in parts:
        out = out + np.asarray(p, dtype=np.float64)
    return out
