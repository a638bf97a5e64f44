"""NF4 codec oracle: codebook, blockwise quantization, double quantization,
dequantization.  TEST INFRASTRUCTURE ONLY (see package docstring).

Arithmetic conventions.  Where the method itself computes in float32 (the
division by the block scale, the int8 step of double quantization, the scale
reconstruction, the weight reconstruction) this module uses NumPy float32
operations, each of which rounds once to nearest-even and never fuses a
multiply with an add.  Where the method fixes no precision (the codebook, the
nearest-level decision, the mean of the scales) it uses exact rationals or
float64 and rounds once at the end.
"""
from __future__ import annotations

import math
from fractions import Fraction
from statistics import NormalDist

import numpy as np

BLOCK = 64          # weights per first-level block ([MC] "2. Double quantization"; [GO] "Idea two")
CHUNK = 256         # first-level scales per second-level scale ([MC] "A worked memory budget")
F32 = np.float32

# ---------------------------------------------------------------------------
# Codebook.  [TT] §5 "NF4": the 16 values sit at quantiles of a standard
# normal; [MC] "1. NormalFloat": 4 bits give 16 codes, arranged for a
# zero-centred normal; [GO] "Idea one": quantile spacing, dense near zero.
#
# Reading (the pages give no formula): the positive half uses 8 quantiles and
# the negative half 7, at probabilities evenly spaced between 1/2 and an outer
# probability NF4_DELTA (the outer quantile of an exactly-1 probability would
# be infinite), plus an exact zero so that zero weights survive quantization.
# All values are divided by the outermost quantile so the codebook spans
# [-1, 1].  NF4_DELTA is the average of 1 - 1/32 and 1 - 1/30: the centre of
# the outermost bin when the probability mass is cut into 2*16 and 2*15 equal
# parts, one per half of the asymmetric code.
# ---------------------------------------------------------------------------
NF4_DELTA = (Fraction(31, 32) + Fraction(29, 30)) / 2


def nf4_levels_f64() -> list:
    """The 16 NF4 levels as float64, ascending (code 0 = -1, code 7 = 0, code 15 = +1)."""
    ppf = NormalDist().inv_cdf
    half = Fraction(1, 2)
    top = ppf(float(NF4_DELTA))
    pos = [ppf(float(half + (NF4_DELTA - half) * Fraction(k, 8))) / top for k in range(1, 9)]
    neg = [-ppf(float(half + (NF4_DELTA - half) * Fraction(k, 7))) / top for k in range(1, 8)]
    return sorted(neg + [0.0] + pos)


def nf4_levels() -> np.ndarray:
    """The codebook stored as float32 (each level rounded once from float64)."""
    return np.array(nf4_levels_f64(), dtype=np.float64).astype(F32)


def nf4_midpoints() -> np.ndarray:
    """Exact midpoints between neighbouring float32 levels, as float64.

    The sum of two neighbouring float32 levels is exact in float64 (their
    exponents differ by at most one, or one of them is zero), and halving is
    exact, so these are the true midpoints.
    """
    q = nf4_levels().astype(np.float64)
    mid = (q[:-1] + q[1:]) / 2.0
    for j in range(15):
        assert Fraction(mid[j]) == (Fraction(float(q[j])) + Fraction(float(q[j + 1]))) / 2
    return mid


def encode(x: np.ndarray) -> np.ndarray:
    """Nearest NF4 level for each normalised value x (float32), ties to the lower level.

    [TT] §2 "Choose a scale, then round": divide by the scale, then round to the
    nearest representable value.  Level j+1 is strictly nearer than level j
    exactly when x lies above their midpoint, so the index of the nearest level
    equals the number of midpoints strictly below x.  A value exactly on a
    midpoint therefore takes the lower level (the pages do not address ties).
    """
    x64 = np.asarray(x, dtype=F32).astype(np.float64)
    return np.searchsorted(nf4_midpoints(), x64, side="left").astype(np.uint8)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, first element in the high nibble ([TT] §3)."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.size % 2:
        c = np.concatenate([c, np.array([7], np.uint8)])
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack_codes(packed: np.ndarray, n: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 15
    return out[:n]


def quantize(w: np.ndarray):
    """Blockwise NF4 quantization of a 1-D float32 array.

    Returns (packed codes uint8[ceil(n/2)], absmax float32[ceil(n/64)]).

    [MC] "1. NormalFloat": weights are split into small blocks, each with its
    own scaling factor; [MC] "2. Double quantization" / [GO] "Idea two": blocks
    of 64 weights; the scale is the block's largest magnitude ([TT] §2: the
    scale is set by the largest absolute weight).  Each weight is divided by its
    block scale (IEEE float32 division) and encoded to the nearest level.

    Readings: a short last block is zero-padded (padding cannot change the
    block's largest magnitude); an all-zero block has scale 0 and every code is
    the zero level (it is divided by 1 instead of 0); an odd n pads the last low
    nibble with the zero-level code 7.
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
    codes = encode(x).reshape(-1)
    packed = pack_codes(codes)[: (n + 1) // 2]
    return packed, absmax


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(F32)


def quantize_bf16(u: np.ndarray):
    """quantize() of bf16 input given as uint16 bit patterns (widened exactly first)."""
    return quantize(bf16_bits_to_f32(u))


# ---------------------------------------------------------------------------
# Double quantization.  [MC] "2. Double quantization": the block scales are
# quantized to 8-bit values, with higher-precision scales shared by larger
# groups; [MC] "A worked memory budget": 256 scales per second-level block;
# [TT] §6: the second stage quantizes the first stage's constants and stores a
# smaller set of higher-level constants; it does not change the 4-bit codes.
# The 8-bit step is [TT] §2's symmetric scheme: scale = largest magnitude / 127,
# divide, round to the nearest integer, -128 unused.  The scales are
# mean-centred first (one mean per tensor), which the 0.127 bits/weight figure
# leaves room for (one extra float32 per tensor, not per chunk).
# ---------------------------------------------------------------------------

def int8_absmax_quantize(c: np.ndarray):
    """Symmetric int8 quantization of one group: returns (int8 codes, float32 step).

    step = fp32(max|c| / 127); q = rint(fp32(c / step)) with ties to even,
    clamped to [-127, 127].  A group of zeros has step 0 and codes 0.
    """
    c = np.asarray(c, dtype=F32)
    m = np.abs(c).max() if c.size else F32(0)
    step = F32(F32(m) / F32(127.0))
    if step == 0:
        return np.zeros(c.shape, np.int8), step
    q = np.rint((c / step).astype(F32))
    return np.clip(q, -127, 127).astype(np.int8), step


def _round_fraction_to_f32(fr: Fraction) -> np.float32:
    """Round a non-negative rational to the nearest float32, ties to even (one rounding)."""
    if fr == 0:
        return F32(0.0)
    num, den = fr.numerator, fr.denominator
    e = num.bit_length() - den.bit_length()          # 2^(e-1) < fr < 2^(e+1)
    if Fraction(2) ** e > fr:
        e -= 1                                        # now 2^e <= fr < 2^(e+1)
    q_exp = max(e - 23, -149)                         # float32 quantum at this magnitude
    sn, sd = (num, den << q_exp) if q_exp >= 0 else (num << -q_exp, den)
    qi, rem = divmod(sn, sd)
    if 2 * rem > sd or (2 * rem == sd and qi & 1):
        qi += 1
    return F32(math.ldexp(qi, q_exp))                 # qi <= 2^24: exact


def exact_mean_f32(a: np.ndarray) -> np.float32:
    """Mean of non-negative float32 values, computed exactly and rounded once to float32.

    Reading: the pages fix no precision for the mean; the exact mean rounded
    once is the one value that does not depend on summation order.  Every
    float32 is an integer multiple of 2^-149, so the sum is an exact integer
    in units of 2^-149.
    """
    a = np.asarray(a, dtype=F32).ravel()
    assert a.size > 0 and np.all(a >= 0) and np.all(np.isfinite(a))
    bits = a.view(np.uint32)
    expo = ((bits >> 23) & 0xFF).astype(np.int64)
    mant = (bits & 0x7FFFFF).astype(np.uint64)
    mant = np.where(expo > 0, mant | np.uint64(0x800000), mant)
    shift = np.maximum(expo, 1) - 1                   # value = mant * 2^(shift - 149)
    total = 0
    for s in np.unique(shift):
        total += int(mant[shift == s].sum(dtype=np.uint64)) << int(s)
    return _round_fraction_to_f32(Fraction(total, a.size << 149))


def double_quant(absmax: np.ndarray):
    """Double quantization of the block scales.

    Returns (qabsmax int8[nb], scale2 float32[ceil(nb/256)], mean float32).
    mean = exact mean of all scales rounded once; c = fp32(a - mean);
    each chunk of 256 consecutive c (the last chunk may be short) goes through
    int8_absmax_quantize.
    """
    a = np.asarray(absmax, dtype=F32).ravel()
    nb = a.size
    mean = exact_mean_f32(a)
    c = (a - mean).astype(F32)
    nch = (nb + CHUNK - 1) // CHUNK
    q = np.empty(nb, np.int8)
    s2 = np.empty(nch, F32)
    for j in range(nch):
        q[j * CHUNK:(j + 1) * CHUNK], s2[j] = int8_absmax_quantize(c[j * CHUNK:(j + 1) * CHUNK])
    return q, s2, mean


def scale_reconstruct(qabsmax: np.ndarray, scale2: np.ndarray, mean) -> np.ndarray:
    """a_hat = fp32(fp32(q * step) + mean): multiply the stored integer by its step
    ([TT] §2, dequantization), then undo the centring.  Two float32 roundings."""
    q = np.asarray(qabsmax, np.int8).astype(F32)
    s2 = np.repeat(np.asarray(scale2, F32), CHUNK)[: q.size]
    return ((q * s2).astype(F32) + F32(mean)).astype(F32)


def dequantize(packed: np.ndarray, qabsmax: np.ndarray, scale2: np.ndarray, mean, n: int,
               out: str = "f32") -> np.ndarray:
    """Reconstruct n weights: w_hat = fp32(level[code] * a_hat[block]).

    [MC] "1. NormalFloat": the codes are dequantized into BF16 before the
    matrix multiplication; [GO] "The core move": each block is dequantized on
    the fly.  out="bf16" returns uint16 bit patterns, rounded to nearest-even
    from the float32 value.
    """
    codes = unpack_codes(packed, n)
    ahat = scale_reconstruct(qabsmax, scale2, mean)
    lv = nf4_levels()
    w = (lv[codes] * np.repeat(ahat, BLOCK)[:n]).astype(F32)
    if out == "f32":
        return w
    if out == "bf16":
        return f32_to_bf16_bits(w)
    raise ValueError(out)


def dequantize_no_dq(packed: np.ndarray, absmax: np.ndarray, n: int) -> np.ndarray:
    """Reconstruction from the unquantized float32 block scales (no double quantization)."""
    codes = unpack_codes(packed, n)
    lv = nf4_levels()
    return (lv[codes] * np.repeat(np.asarray(absmax, F32), BLOCK)[:n]).astype(F32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.asarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)
