"""Pins of the oracle's 4-bit codebook variants (oracle.codebooks): the level
tables against their definitions, the nearest-level encoder against exact
brute force, the generic NF4 path against the NF4 codec, reconstruction error
bounds, and the pages' qualitative claim that NF4 suits normally distributed
weights better than evenly spaced or FP4 values ([TT] §5 "NF4"; [MC] "1.
NormalFloat"; [GO] "Idea one")."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import codebooks as cbk


def test_int4_levels_are_the_symmetric_integer_grid():
    lv = cbk.levels("int4")
    for c in range(16):
        assert lv[c] == np.float32(float(Fraction(c - 8, 7)))
    assert lv[1] == -1 and lv[15] == 1 and lv[8] == 0 and cbk.zero_code("int4") == 8
    assert np.array_equal(lv[1:], -lv[1:][::-1])


def test_fp4_levels_are_the_e2m1_values_over_six():
    lv = cbk.levels("fp4")
    mags = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    vals = sorted({s * m for m in mags for s in (1, -1)})
    assert len(vals) == 15
    for c in range(1, 16):
        assert lv[c] == np.float32(vals[c - 1] / 6.0)
    assert lv[0] < -1 and lv[1] == -1 and lv[15] == 1 and cbk.zero_code("fp4") == 8


@pytest.mark.parametrize("cb", cbk.CODEBOOKS)
def test_encoder_is_the_nearest_level_with_ties_down(cb):
    lv = [Fraction(float(x)) for x in cbk.levels(cb)]
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.uniform(-1, 1, 3000).astype(np.float32),
                         np.array([-1, 1, 0, -0.0], np.float32),
                         # float32 values next to every midpoint
                         np.array([np.nextafter(np.float32(float((lv[j] + lv[j + 1]) / 2)), d)
                                   for j in range(15) for d in (-2, 2)], np.float32)])
    xs = xs[np.abs(xs) <= 1]
    got = cbk.encode(xs, cb)
    for x, c in zip(xs, got):
        fx = Fraction(float(x))
        d = [abs(fx - l) for l in lv]
        best = min(range(16), key=lambda j: (d[j], j))   # nearest, ties to the lower level
        assert c == best, (cb, float(x), int(c), best)


def test_generic_path_reproduces_the_nf4_codec():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal(64 * 37 + 5) * 0.02).astype(np.float32)
    p1, a1 = oracle.quantize(w)
    p2, a2 = cbk.quantize(w, "nf4")
    assert np.array_equal(p1, p2) and np.array_equal(a1, a2)
    q, s2, mean = oracle.double_quant(a1)
    assert np.array_equal(cbk.dequantize(p2, q, s2, mean, w.size, "nf4"),
                          oracle.dequantize(p1, q, s2, mean, w.size))
    assert np.array_equal(cbk.dequantize_no_dq(p2, a2, w.size, "nf4"), oracle.dequantize_no_dq(p1, a1, w.size))


@pytest.mark.parametrize("cb", cbk.CODEBOOKS)
def test_no_dq_error_is_at_most_half_the_widest_gap(cb):
    rng = np.random.default_rng(7)
    w = (rng.standard_normal(64 * 200) * 0.02).astype(np.float32)
    w[::97] *= 10
    lv = cbk.levels(cb).astype(np.float64)
    gap = np.max(np.diff(lv[lv >= -1]))          # the levels a value in [-1, 1] can take
    _, a = cbk.quantize(w, cb)
    err = np.abs(cbk.reconstruction(w, cb, dq=False).astype(np.float64) - w)
    amax = np.repeat(a.astype(np.float64), 64)[: w.size]
    assert np.all(err <= (gap / 2) * amax * (1 + 1e-6) + 1e-12)
    # the block's absmax element is reproduced exactly (levels -1 and +1 are exact)
    blocks = w.reshape(-1, 64)
    i = np.argmax(np.abs(blocks), axis=1)
    rec = cbk.reconstruction(w, cb, dq=False).reshape(-1, 64)
    assert np.array_equal(rec[np.arange(len(i)), i], blocks[np.arange(len(i)), i])


def test_odd_length_pads_with_the_zero_code():
    for cb in cbk.CODEBOOKS:
        p, _ = cbk.quantize(np.array([0.5, -0.25, 0.1], np.float32), cb)
        assert p[-1] & 15 == cbk.zero_code(cb)


def test_nf4_has_the_lowest_error_on_normal_weights():
    rng = np.random.default_rng(11)
    w = rng.standard_normal(64 * 4000).astype(np.float32)
    mse = {cb: cbk.reconstruction_mse(w, cb, dq=False) for cb in cbk.CODEBOOKS}
    assert mse["nf4"] < mse["int4"] and mse["nf4"] < mse["fp4"], mse
    # double quantization adds little on top ([MC] "2. Double quantization")
    for cb in cbk.CODEBOOKS:
        assert cbk.reconstruction_mse(w, cb, dq=True) < 1.02 * mse[cb]
