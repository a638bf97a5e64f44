"""Pins for the oracle's blockwise NF4 quantization, double quantization and
dequantization: brute force with exact rationals, round trips, the worked INT8
example printed on the pages, tie and padding cases, and error bounds."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

F32 = np.float32


def exact_nearest(x: float, levels) -> int:
    """Brute force: index of the nearest level by exact rational distance, ties to lower."""
    fx = Fraction(float(x))
    best, bestd = None, None
    for j, q in enumerate(levels):
        d = abs(fx - Fraction(float(q)))
        if bestd is None or d < bestd:
            best, bestd = j, d
    return best


def f32_neighbours(x: float, k: int) -> np.ndarray:
    """2k+1 consecutive float32 values centred on float32(x)."""
    c = np.float32(x)
    out = [c]
    lo = hi = c
    for _ in range(k):
        lo = np.nextafter(lo, np.float32(-np.inf))
        hi = np.nextafter(hi, np.float32(np.inf))
        out += [lo, hi]
    return np.array(out, dtype=F32)


def test_encode_exact_near_every_midpoint():
    lv = oracle.nf4_levels()
    mid = oracle.nf4_midpoints()
    xs = np.concatenate([f32_neighbours(m, 48) for m in mid])
    got = oracle.encode(xs)
    want = np.array([exact_nearest(x, lv) for x in xs])
    assert np.array_equal(got, want)


def test_encode_random_and_special_values_vs_fp64_argmin():
    rng = np.random.default_rng(7)
    xs = np.concatenate([
        rng.uniform(-1, 1, 1 << 18).astype(F32),
        np.array([0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 1e-38, -1e-38], F32),
        oracle.nf4_levels(),
    ])
    lv = oracle.nf4_levels().astype(np.float64)
    # np.argmin returns the first minimum, i.e. ties go to the lower level.  The
    # differences are exact in float64 near the midpoints, where ties can occur.
    want = np.argmin(np.abs(xs.astype(np.float64)[:, None] - lv[None, :]), axis=1)
    assert np.array_equal(oracle.encode(xs), want)


def test_encode_ties_go_to_lower_level():
    lv = oracle.nf4_levels()
    mid = oracle.nf4_midpoints()
    for j in (2, 6, 7, 14):
        assert oracle.encode(np.array([mid[j]], F32))[0] == j
        assert oracle.encode(np.array([np.nextafter(F32(mid[j]), F32(2))], F32))[0] == j + 1
    assert oracle.encode(lv).tolist() == list(range(16))


def brute_quantize(w: np.ndarray):
    """Element by element: block absmax, IEEE float32 divide, exact nearest level."""
    lv = oracle.nf4_levels()
    n = w.size
    codes, absmax = [], []
    for b in range(0, n, 64):
        blk = [F32(v) for v in w[b:b + 64]]
        a = max(abs(v) for v in blk)
        absmax.append(F32(a))
        for v in blk:
            x = F32(v) / F32(a) if a > 0 else F32(0.0)
            codes.append(exact_nearest(x, lv))
        codes += [7] * (64 - len(blk)) if b + 64 > n else []
    codes = codes[:n]
    if n % 2:
        codes.append(7)
    packed = [(codes[i] << 4) | codes[i + 1] for i in range(0, len(codes), 2)]
    return np.array(packed, np.uint8), np.array(absmax, F32)


@pytest.mark.parametrize("n,seed", [(64, 0), (130, 1), (1, 2), (63, 3), (257, 4), (640, 5)])
def test_quantize_matches_brute_force(n, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(n) * 0.02).astype(F32)
    if n > 10:
        w[3] = F32(0.5)                       # an outlier in the first block
    p, a = oracle.quantize(w)
    bp, ba = brute_quantize(w)
    assert np.array_equal(a.view(np.uint32), ba.view(np.uint32))
    assert np.array_equal(p, bp)


@pytest.mark.parametrize("a", [1.0, 0.02, 0.0371, 3.5e-30, 2.0 ** -126, 1e30, 0.0625])
def test_round_trip_of_every_level_times_absmax(a):
    """A block holding fp32(level_i * a) for all i (including +a itself) encodes to i
    and, without double quantization, decodes to the identical float32 bits."""
    lv = oracle.nf4_levels()
    a = F32(a)
    vals = (lv * a).astype(F32)
    w = np.concatenate([vals, vals[::-1], vals, vals[::-1]])       # one 64-block
    p, am = oracle.quantize(w)
    assert am[0] == a
    codes = oracle.unpack_codes(p, 64)
    assert codes.tolist() == (list(range(16)) + list(range(15, -1, -1))) * 2
    back = oracle.dequantize_no_dq(p, am, 64)
    assert np.array_equal(back.view(np.uint32), w.view(np.uint32))


def test_zero_block_negative_zero_and_padding():
    w = np.zeros(64 + 5, F32)
    w[64:] = [0.3, -0.3, -0.0, 0.0, 0.15]
    w[1] = -0.0
    p, a = oracle.quantize(w)
    assert a[0] == 0 and a[1] == F32(0.3)
    codes = oracle.unpack_codes(p, w.size)
    assert np.all(codes[:64] == 7)                                  # all-zero block -> zero level
    assert codes[64:].tolist() == [15, 0, 7, 7, oracle.encode(np.array([F32(0.15) / F32(0.3)]))[0]]
    assert p.size == 35 and (p[-1] & 15) == 7                      # odd n: pad nibble is code 7
    assert oracle.quantize(np.array([0.25, -0.25, 0.0], F32))[0].tolist() == [0xF0, 0x77]


def test_int8_worked_example(golden):
    """The symmetric INT8 example of the pages, through the oracle's int8 step."""
    g = golden("int8_worked_example.txt")
    grp = np.array([g["group_absmax"], -g["group_absmax"], g["weight"], g["example_value"] + 0.004], F32)
    q, step = oracle.int8_absmax_quantize(grp)
    assert abs(float(step) - g["step"]) < 1e-9
    assert F32(grp[2]) / step == pytest.approx(g["scaled"], abs=1e-5)
    assert int(q[2]) == g["stored"] and int(q[0]) == 127 and int(q[1]) == -127
    recovered = float(F32(q[2]) * step)
    assert recovered == pytest.approx(g["recovered"], abs=1e-6)
    assert abs(recovered - g["weight"]) == pytest.approx(g["error"], abs=1e-6)
    assert int(q[3]) == g["example_integer"]
    assert float(F32(q[3]) * step) == pytest.approx(g["example_value"], abs=1e-6)
    _, step_out = oracle.int8_absmax_quantize(np.array([g["outlier_absmax"], 0.5], F32))
    assert float(step_out) == pytest.approx(g["outlier_step"], abs=1e-7)


def test_int8_zero_group_and_range():
    q, step = oracle.int8_absmax_quantize(np.zeros(5, F32))
    assert step == 0 and np.all(q == 0)
    rng = np.random.default_rng(3)
    c = rng.standard_normal(256).astype(F32)
    q, step = oracle.int8_absmax_quantize(c)
    assert q.min() >= -127 and np.abs(q).max() == 127                # -128 unused, range used
    assert np.all(np.abs(q.astype(np.float64) * float(step) - c) <= float(step) * (0.5 + 1e-6))


def _round_to_f32_by_neighbours(fr: Fraction) -> np.float32:
    """Independent rounding: pick the closest of float32(float(fr)) and its neighbours,
    ties to the even significand."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - fr), int(np.array(v).view(np.uint32)) & 1))
    return best


@pytest.mark.parametrize("seed", range(6))
def test_exact_mean_vs_fractions(seed):
    rng = np.random.default_rng(seed)
    n = [1, 7, 256, 1000, 4099, 3][seed]
    a = np.abs(rng.standard_normal(n) * [0.02, 1e-3, 5.0, 1e-38, 1e30, 0.1][seed]).astype(F32)
    if seed == 3:
        a[::3] = F32(1e-45)                                          # denormals
    exact = sum(Fraction(float(v)) for v in a) / n
    assert oracle.exact_mean_f32(a) == _round_to_f32_by_neighbours(exact)


def test_exact_mean_ties_to_even():
    one = F32(1.0)
    up = np.nextafter(one, F32(2))
    up2 = np.nextafter(up, F32(2))
    assert oracle.exact_mean_f32(np.array([one, up], F32)) == one      # 1 + 2^-24: tie -> even (1.0)
    # 1 + 1.5 * 2^-23 lies halfway between 1 + 2^-23 (odd) and 1 + 2^-22 (even)
    assert oracle.exact_mean_f32(np.array([up, up2], F32)) == up2
    # a sum that is not representable in float64 either: the mean is still exact
    a = np.array([1e30, 1e-30, 1e-30], F32)
    assert oracle.exact_mean_f32(a) == _round_to_f32_by_neighbours(sum(Fraction(float(v)) for v in a) / 3)


@pytest.mark.parametrize("nb", [1, 255, 256, 257, 600])
def test_double_quant_structure_and_error_bound(nb):
    rng = np.random.default_rng(nb)
    a = np.abs(rng.standard_normal(nb) * 0.02).astype(F32) + F32(0.01)
    q, s2, mean = oracle.double_quant(a)
    assert q.dtype == np.int8 and q.size == nb
    assert s2.dtype == np.float32 and s2.size == (nb + 255) // 256
    assert mean == oracle.exact_mean_f32(a)
    c = (a - mean).astype(F32)
    for j in range(s2.size):
        cj = c[j * 256:(j + 1) * 256]
        qj = q[j * 256:(j + 1) * 256]
        assert s2[j] == F32(np.abs(cj).max() / F32(127))
        if s2[j] == 0:                                               # a single scale: c == 0
            assert np.all(qj == 0)
            continue
        assert np.abs(qj).max() == 127 and qj.min() >= -127
        k = np.argmax(np.abs(cj))
        assert qj[k] == (127 if cj[k] > 0 else -127)                  # the extreme maps to +-127
        assert np.all(np.sign(qj[np.abs(cj) > s2[j]]) == np.sign(cj[np.abs(cj) > s2[j]]))
    ahat = oracle.scale_reconstruct(q, s2, mean)
    step = np.repeat(s2, 256)[:nb].astype(np.float64)
    err = np.abs(ahat.astype(np.float64) - a.astype(np.float64))
    assert np.all(err <= step * 0.5 + 4 * np.spacing(np.maximum(np.abs(a), np.abs(ahat))).astype(np.float64))


def test_double_quant_constant_scales():
    a = np.full(300, F32(0.0421), F32)
    q, s2, mean = oracle.double_quant(a)
    assert mean == F32(0.0421) and np.all(s2 == 0) and np.all(q == 0)
    assert np.all(oracle.scale_reconstruct(q, s2, mean) == F32(0.0421))


def test_double_quant_leaves_codes_unchanged():
    """[TT] §6: double quantization does not change the 4-bit codes.  The codes come
    from the float32 block scales, before any scale is quantized."""
    w = (np.random.default_rng(11).standard_normal(64 * 300) * 0.02).astype(F32)
    p, a = oracle.quantize(w)
    q, s2, mean = oracle.double_quant(a)
    p2, _ = oracle.quantize(w)
    assert np.array_equal(p, p2)
    ahat = oracle.scale_reconstruct(q, s2, mean)
    d = oracle.dequantize(p, q, s2, mean, w.size)
    lv = oracle.nf4_levels()
    assert np.array_equal(d, (lv[oracle.unpack_codes(p, w.size)] * np.repeat(ahat, 64)).astype(F32))


def test_dequantize_zero_code_and_bf16():
    p = np.array([0x77, 0xF0], np.uint8)
    q = np.array([5], np.int8)
    s2 = np.array([0.001], F32)
    mean = F32(0.05)
    d = oracle.dequantize(p, q, s2, mean, 4)
    ahat = F32(F32(F32(5) * F32(0.001)) + mean)
    assert d.tolist() == [0.0, 0.0, float(ahat), float(-ahat)]
    b = oracle.dequantize(p, q, s2, mean, 4, out="bf16")
    assert b.dtype == np.uint16 and b[0] == 0 and b[2] == oracle.f32_to_bf16_bits(np.array([ahat]))[0]


def test_bf16_rounding_vs_torch_and_ties():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(1 << 16).astype(F32) * 0.03,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.4e38, 1e-40], F32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(x), ref)
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert oracle.f32_to_bf16_bits(np.array([1.0 + 2 ** -8], F32))[0] == 0x3F80
    assert oracle.f32_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8], F32))[0] == 0x3F82


def _bf16_value(u: int) -> float:
    """The value of a bf16 bit pattern from its fields ([TT] §1 "FP32, FP16, BF16,
    and FP8": 1 sign bit, 8 exponent bits with float32's bias, 7 fraction bits)."""
    sign = -1.0 if u >> 15 else 1.0
    e, f = (u >> 7) & 0xFF, u & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


def test_bf16_widening_every_pattern():
    """oracle.bf16_bits_to_f32 against the field definition for all 65,536 patterns
    (NaNs: still NaN, sign kept) and against torch's bfloat16 -> float32 widening."""
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_bits_to_f32(u)
    assert got.dtype == np.float32 and got.shape == u.shape
    ref = np.array([_bf16_value(int(v)) for v in u], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].astype(np.float64), ref[~nan])
    assert np.array_equal(np.signbit(got), u >= 0x8000)
    t = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(t.view(np.uint32), got.view(np.uint32))


def test_bf16_widening_hand_built():
    cases = {0x0000: 0.0, 0x8000: -0.0, 0x0001: math.ldexp(1.0, -133), 0x807F: -math.ldexp(127.0, -133),
             0x0080: math.ldexp(1.0, -126), 0x3F80: 1.0, 0xBF80: -1.0, 0x4049: 3.140625,
             0x7F7F: math.ldexp(255.0, 120), 0xFF7F: -math.ldexp(255.0, 120), 0x7F80: math.inf, 0xFF80: -math.inf}
    u = np.array(list(cases), dtype=np.uint16)
    got = oracle.bf16_bits_to_f32(u)
    for v, g in zip(cases.values(), got):
        assert g == v and math.copysign(1.0, g) == math.copysign(1.0, v)


def test_quantize_bf16_matches_widened_input():
    """quantize_bf16 is quantize() of the widened values: checked on bf16 patterns whose
    values are fixed by hand (the codebook ends, zero, a level times a power of two) and
    on random patterns widened by torch (not by the oracle)."""
    # one block: 1.0, -1.0, +0, -0, 0.5, then zeros; absmax 1, codes 15, 0, 7, 7 and
    # the nearest level to 0.5 (found by brute force over the levels)
    u = np.zeros(64, np.uint16)
    u[:5] = [0x3F80, 0xBF80, 0x0000, 0x8000, 0x3F00]
    packed, absmax = oracle.quantize_bf16(u)
    lv = oracle.nf4_levels().astype(np.float64)
    c_half = int(np.argmin(np.abs(lv - 0.5)))
    codes = oracle.unpack_codes(packed, 64)
    assert absmax[0] == 1.0
    assert list(codes[:5]) == [15, 0, 7, 7, c_half] and set(codes[5:]) == {7}
    rng = np.random.default_rng(7)
    r = rng.integers(0, 1 << 16, size=4096).astype(np.uint16)
    r = r[((r >> 7) & 0xFF) != 0xFF]  # finite values only ([TT] weights are finite)
    widened = torch.from_numpy(r.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    p1, a1 = oracle.quantize_bf16(r)
    p2, a2 = oracle.quantize(widened)
    assert np.array_equal(p1, p2) and np.array_equal(a1.view(np.uint32), a2.view(np.uint32))
