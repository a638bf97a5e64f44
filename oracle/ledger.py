"""Storage ledger of the oracle's own NF4 formats.  TEST INFRASTRUCTURE ONLY.

[TL] "02 · The mechanism": raw storage is parameter count x bits / 8 bytes,
plus quantization metadata; GB divides by 10^9.  The sizes here are measured on
the arrays that oracle.nf4 actually produces, so the ledger pins the formats
(4-bit codes two per byte, one scale per 64 weights, int8 scales with one
float32 step per 256 scales and one float32 mean per tensor).
"""
from __future__ import annotations

import numpy as np

from .nf4 import double_quant, quantize


def storage_bytes(n: int, double_quant_on: bool = True, seed: int = 0) -> dict:
    """Byte sizes of each stored part for an n-weight tensor (measured on real arrays)."""
    w = np.random.default_rng(seed).standard_normal(n).astype(np.float32)
    packed, absmax = quantize(w)
    parts = {"codes": packed.nbytes}
    if double_quant_on:
        q, s2, mean = double_quant(absmax)
        parts.update(qabsmax=q.nbytes, scale2=s2.nbytes, mean=np.float32(mean).nbytes)
    else:
        parts.update(absmax=absmax.nbytes)
    return parts


def storage_bits_per_weight(n: int, double_quant_on: bool = True, include_codes: bool = False,
                            include_mean: bool = False) -> float:
    """Scale-metadata bits per weight (optionally with the 4-bit codes / the tensor mean)."""
    parts = storage_bytes(n, double_quant_on)
    total = sum(v for k, v in parts.items()
                if (include_codes or k != "codes") and (include_mean or k != "mean"))
    return 8.0 * total / n


def lora_param_count(h: int, o: int, r: int) -> int:
    """Trainable parameters of one adapter: L1 (h x r) plus L2 (r x o)."""
    return h * r + r * o
