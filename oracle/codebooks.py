"""4-bit codebook variants the pages compare with NF4.  TEST INFRASTRUCTURE ONLY.

[MC] "1. NormalFloat" and [TT] §5 "NF4" contrast NF4 with evenly spaced 4-bit
values; [MC] "What the experiments establish" (Fig. 3) and [GO] "Idea one"
compare NF4 with FP4; [TT] §2 "Choose a scale, then round" gives the
symmetric absmax scheme that an integer 4-bit code uses; [MC] "2. Double
quantization" / [TT] §6 make double quantization of the block scales an
option on top of any of them.

Every variant keeps the NF4 storage: blocks of 64 weights, the block's largest
magnitude as its scale, x = fp32(w / absmax), a code per weight (two per byte,
first in the high nibble), and w_hat = fp32(level[code] * scale), where the
scale is either the float32 absmax itself (no double quantization) or
a_hat = fp32(fp32(q * s2) + mean) (double quantization).  A code is the index
of its level in an ascending 16-entry table, chosen as the nearest level with
ties to the lower one (the NF4 rule).

Readings (the pages fix none of these tables):
- "int4": the symmetric absmax integer grid at 4 bits, levels q / 7 for
  q = -8..7 (code = q + 8).  |x| <= 1, so q = -8 is never chosen, as -128 is
  never chosen by the int8 scheme.
- "fp4": the FP4 values of the common E2M1 layout, magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}, divided by 6 so that the largest is 1; the
  15 distinct values sit at codes 1..15 and code 0 holds an unused -1.5.
- "nf4": the NF4 codebook of oracle.nf4.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .nf4 import BLOCK, F32, double_quant, nf4_levels, pack_codes, scale_reconstruct, unpack_codes

CODEBOOKS = ("nf4", "int4", "fp4")
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def levels_fraction(cb: str) -> list:
    """The 16 levels as exact rationals (nf4: its float32 values), ascending."""
    if cb == "nf4":
        return [Fraction(float(x)) for x in nf4_levels()]
    if cb == "int4":
        return [Fraction(q, 7) for q in range(-8, 8)]
    if cb == "fp4":
        mags = [Fraction(m) / 6 for m in E2M1_MAGNITUDES]
        vals = sorted(set([-m for m in mags] + mags))          # 15 distinct values
        return [Fraction(-3, 2)] + vals
    raise ValueError(cb)


def levels(cb: str) -> np.ndarray:
    """The 16 levels as float32 (each rational rounded once)."""
    return np.array([float(f) for f in levels_fraction(cb)], dtype=np.float64).astype(F32)


def zero_code(cb: str) -> int:
    return int(np.flatnonzero(levels(cb) == 0)[0])


def midpoints(cb: str) -> np.ndarray:
    """Exact midpoints of neighbouring float32 levels, as float64 (exact: see oracle.nf4)."""
    q = levels(cb).astype(np.float64)
    mid = (q[:-1] + q[1:]) / 2.0
    for j in range(15):
        assert Fraction(mid[j]) == (Fraction(float(q[j])) + Fraction(float(q[j + 1]))) / 2
    return mid


def encode(x: np.ndarray, cb: str) -> np.ndarray:
    """Nearest level of the float32 value x, ties to the lower level: the number of
    midpoints strictly below x."""
    x64 = np.asarray(x, dtype=F32).astype(np.float64)
    return np.searchsorted(midpoints(cb), x64, side="left").astype(np.uint8)


def quantize(w: np.ndarray, cb: str):
    """Blockwise quantization of a 1-D float32 array with codebook cb.

    Returns (packed codes uint8[ceil(n/2)], absmax float32[ceil(n/64)]); the same
    readings as oracle.nf4.quantize (short last block zero-padded, an all-zero block
    has scale 0 and every code is the zero level, odd n pads the last low nibble
    with the zero level's code).
    """
    w = np.asarray(w, dtype=F32).ravel()
    n = w.size
    nb = (n + BLOCK - 1) // BLOCK
    wp = np.zeros(nb * BLOCK, dtype=F32)
    wp[:n] = w
    blocks = wp.reshape(nb, BLOCK)
    absmax = np.abs(blocks).max(axis=1).astype(F32)
    divisor = np.where(absmax > 0, absmax, F32(1.0)).astype(F32)
    x = (blocks / divisor[:, None]).astype(F32)
    codes = encode(x, cb).reshape(-1)[:n]
    if n % 2:
        codes = np.concatenate([codes, np.array([zero_code(cb)], np.uint8)])
    packed = ((codes[0::2] << 4) | codes[1::2]).astype(np.uint8)
    return packed, absmax


def dequantize(packed: np.ndarray, qabsmax, scale2, mean, n: int, cb: str) -> np.ndarray:
    """w_hat = fp32(level[code] * a_hat) with double-quantized scales."""
    codes = unpack_codes(packed, n)
    ahat = scale_reconstruct(qabsmax, scale2, mean)
    return (levels(cb)[codes] * np.repeat(ahat, BLOCK)[:n]).astype(F32)


def dequantize_no_dq(packed: np.ndarray, absmax: np.ndarray, n: int, cb: str) -> np.ndarray:
    """w_hat = fp32(level[code] * absmax) from the float32 block scales."""
    codes = unpack_codes(packed, n)
    return (levels(cb)[codes] * np.repeat(np.asarray(absmax, F32), BLOCK)[:n]).astype(F32)


def reconstruction(w: np.ndarray, cb: str, dq: bool) -> np.ndarray:
    """Quantize then dequantize (with or without double quantization)."""
    w = np.asarray(w, dtype=F32).ravel()
    p, a = quantize(w, cb)
    if dq:
        q, s2, mean = double_quant(a)
        return dequantize(p, q, s2, mean, w.size, cb)
    return dequantize_no_dq(p, a, w.size, cb)


def reconstruction_mse(w: np.ndarray, cb: str, dq: bool) -> float:
    """Mean squared reconstruction error in float64."""
    w = np.asarray(w, dtype=F32).ravel()
    d = reconstruction(w, cb, dq).astype(np.float64) - w.astype(np.float64)
    return float(np.mean(d * d))


__all__ = ["CODEBOOKS", "levels", "levels_fraction", "zero_code", "midpoints", "encode", "quantize",
           "dequantize", "dequantize_no_dq", "reconstruction", "reconstruction_mse", "pack_codes"]
