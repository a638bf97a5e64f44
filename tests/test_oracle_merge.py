"""Pins of the oracle's adapter merge ([TT] §11 "Saving, Loading, and Merging QLoRA
Adapters"): W' = W_hat + s * L1 L2 in [o][h] storage, float32 steps."""
import numpy as np
import pytest

import oracle
import workloads as wl


def _problem(h, o, r, seed):
    w, l1, l2, _, _ = wl.small_linear(h, o, r, 4, seed=seed)
    p, a = oracle.quantize(w.numpy().ravel())
    q, s2, mean = oracle.double_quant(a)
    L1 = None if l1 is None else l1.float().numpy()
    L2 = None if l2 is None else l2.float().numpy()
    return p, q, s2, mean, L1, L2


def test_no_adapter_or_zero_scale_is_the_dequantized_weight():
    p, q, s2, mean, L1, L2 = _problem(128, 64, 8, 1)
    wh = oracle.dequantized_weight(p, q, s2, mean, 128, 64)
    assert np.array_equal(oracle.merged_weight(p, q, s2, mean, 128, 64, None, None, 2.0), wh)
    assert np.array_equal(oracle.merged_weight(p, q, s2, mean, 128, 64, L1, L2, 0.0).view(np.uint32),
                          (wh + np.float32(0.0)).view(np.uint32))


@pytest.mark.parametrize("r,s", [(1, 2.0), (8, 0.25), (24, 1.5)])
def test_matches_exact_merge_within_float32_summation_bound(r, s):
    h, o = 192, 128
    p, q, s2, mean, L1, L2 = _problem(h, o, r, 10 + r)
    wh = oracle.dequantized_weight(p, q, s2, mean, h, o).astype(np.float64)
    got = oracle.merged_weight(p, q, s2, mean, h, o, L1, L2, s).astype(np.float64)
    prod = (L1.astype(np.float64) @ L2.astype(np.float64)).T          # [o][h]: transposed adapter product
    exact = wh + s * prod
    mag = np.abs(wh) + abs(s) * (np.abs(L1.astype(np.float64)) @ np.abs(L2.astype(np.float64))).T
    bound = (r + 3) * 2.0 ** -24 * mag + 1e-45
    assert np.all(np.abs(got - exact) <= bound)
    # a dropped, transposed or mis-scaled term would exceed the bound by orders of magnitude
    assert np.max(np.abs(prod)) * abs(s) > 1e3 * np.max(bound)


def test_merged_weight_reproduces_the_adapter_forward():
    h, o, r, s = 128, 192, 8, 2.0
    p, q, s2, mean, L1, L2 = _problem(h, o, r, 3)
    x = np.random.default_rng(0).standard_normal((5, h))
    wm = oracle.merged_weight(p, q, s2, mean, h, o, L1, L2, s)
    wh = oracle.dequantized_weight(p, q, s2, mean, h, o)
    y_merged, _ = oracle.linear_fwd(wm, x, None, None, s)
    y_adapter, _ = oracle.linear_fwd(wh, x, L1, L2, s)
    assert np.allclose(y_merged, y_adapter, rtol=1e-5, atol=1e-5 * np.abs(y_adapter).max())


def test_requantizing_an_unmodified_merge_reproduces_the_codes():
    """Each block holds a +-1 code (its absmax element), so re-quantizing W_hat gives the same
    codes and, as new absmax, the rebuilt scale a_hat of every block."""
    h, o = 256, 64
    p, q, s2, mean, _, _ = _problem(h, o, 0, 7)
    wm = oracle.merged_weight(p, q, s2, mean, h, o, None, None, 1.0)
    p2, a2 = oracle.quantize(wm.ravel())
    assert np.array_equal(p2, p)
    assert np.array_equal(a2.view(np.uint32), np.abs(oracle.scale_reconstruct(q, s2, mean)).view(np.uint32))
