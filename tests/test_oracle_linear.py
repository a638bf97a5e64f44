"""Pins for the oracle's LoRA linear layer: closed forms on one-hot inputs,
special cases that reduce to a plain matmul, central finite differences of the
backward, and the adjoint identities that tie the backward to the forward."""
import numpy as np
import pytest

import oracle


def problem(m, h, o, r, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((o, h)) * 0.02).astype(np.float32)
    x = rng.standard_normal((m, h))
    l1 = rng.standard_normal((h, r)) * 0.1 if r else None
    l2 = rng.standard_normal((r, o)) * 0.1 if r else None
    dy = rng.standard_normal((m, o))
    return w, x, l1, l2, dy


def test_one_hot_rows_give_weight_rows():
    """X = e_i picks row i of the pages' h x o weight (column i of the [o][h] buffer)
    plus s * L1[i] L2 — catches a transposed operand or a dropped term."""
    h, o, r, s = 64, 5, 3, 0.75
    w, _, l1, l2, _ = problem(1, h, o, r, 1)
    for i in (0, 17, 63):
        x = np.zeros((1, h))
        x[0, i] = 1.0
        y, t = oracle.linear_fwd(w, x, l1, l2, s)
        assert np.allclose(y[0], w[:, i].astype(np.float64) + s * (l1[i] @ l2), rtol=0, atol=1e-15)
        assert np.allclose(t[0], l1[i], rtol=0, atol=0)


def test_no_adapter_is_plain_matmul():
    w, x, l1, l2, dy = problem(4, 128, 7, 2, 2)
    y0, t0 = oracle.linear_fwd(w, x, None, None, 2.0)
    assert t0 is None
    assert np.allclose(y0, np.matmul(x, w.astype(np.float64).T), rtol=1e-14, atol=1e-14)
    y_s0, _ = oracle.linear_fwd(w, x, l1, l2, 0.0)
    assert np.array_equal(y_s0, y0)
    dx0, a, b = oracle.linear_bwd(w, x, dy, None, None, 2.0)
    assert a is None and b is None
    assert np.allclose(dx0, np.matmul(dy, w.astype(np.float64)), rtol=1e-14, atol=1e-14)


def test_zero_weight_isolates_adapter():
    w, x, l1, l2, dy = problem(3, 64, 6, 4, 3)
    y, _ = oracle.linear_fwd(np.zeros_like(w), x, l1, l2, 1.5)
    assert np.allclose(y, 1.5 * np.matmul(np.matmul(x, l1), l2), rtol=1e-13, atol=1e-14)


def test_triple_loop_brute_force():
    m, h, o, r, s = 3, 64, 5, 2, 1.25
    w, x, l1, l2, dy = problem(m, h, o, r, 4)
    y, _ = oracle.linear_fwd(w, x, l1, l2, s)
    for i in range(m):
        for j in range(o):
            acc = 0.0
            for k in range(h):
                acc += x[i, k] * float(w[j, k])
                for q in range(r):
                    acc += s * x[i, k] * l1[k, q] * l2[q, j]
            assert abs(acc - y[i, j]) < 1e-12


@pytest.mark.parametrize("seed", [5, 6])
def test_backward_matches_central_differences(seed):
    """f = <dY, Y(X, L1, L2)> is linear in each argument, so central differences are
    exact up to rounding; its partial derivatives are dX, dL1, dL2."""
    m, h, o, r, s = 4, 64, 9, 3, 0.5
    w, x, l1, l2, dy = problem(m, h, o, r, seed)
    dx, dl1, dl2 = oracle.linear_bwd(w, x, dy, l1, l2, s)

    def f(x_, l1_, l2_):
        return float(np.sum(dy * oracle.linear_fwd(w, x_, l1_, l2_, s)[0]))

    rng = np.random.default_rng(seed)
    eps = 1e-3
    for _ in range(6):
        i, k = rng.integers(m), rng.integers(h)
        xp, xm = x.copy(), x.copy()
        xp[i, k] += eps
        xm[i, k] -= eps
        assert (f(xp, l1, l2) - f(xm, l1, l2)) / (2 * eps) == pytest.approx(dx[i, k], rel=1e-8, abs=1e-10)
        k, q = rng.integers(h), rng.integers(r)
        ap, am = l1.copy(), l1.copy()
        ap[k, q] += eps
        am[k, q] -= eps
        assert (f(x, ap, l2) - f(x, am, l2)) / (2 * eps) == pytest.approx(dl1[k, q], rel=1e-8, abs=1e-10)
        q, j = rng.integers(r), rng.integers(o)
        bp, bm = l2.copy(), l2.copy()
        bp[q, j] += eps
        bm[q, j] -= eps
        assert (f(x, l1, bp) - f(x, l1, bm)) / (2 * eps) == pytest.approx(dl2[q, j], rel=1e-8, abs=1e-10)


def test_adjoint_identities():
    m, h, o, r, s = 8, 128, 16, 4, 2.0
    w, x, l1, l2, dy = problem(m, h, o, r, 9)
    y, _ = oracle.linear_fwd(w, x, l1, l2, s)
    y_base, _ = oracle.linear_fwd(w, x, None, None, s)
    dx, dl1, dl2 = oracle.linear_bwd(w, x, dy, l1, l2, s)
    lhs = np.sum(dy * y)
    assert np.sum(dx * x) == pytest.approx(lhs, rel=1e-12)
    lora = np.sum(dy * (y - y_base))
    assert np.sum(dl1 * l1) == pytest.approx(lora, rel=1e-10)
    assert np.sum(dl2 * l2) == pytest.approx(lora, rel=1e-10)


def test_dequantized_weight_layout():
    """The [o][h] buffer's 64-blocks run along h: one block per 64 inputs of one output."""
    h, o = 128, 3
    w = np.zeros((o, h), np.float32)
    w[1, 64:] = 0.5                            # second block of output row 1
    p, a = oracle.quantize(w.ravel())
    assert a.tolist() == [0, 0, 0, 0.5, 0, 0]
    q, s2, mean = oracle.double_quant(a)
    wd = oracle.dequantized_weight(p, q, s2, mean, h, o)
    assert wd.shape == (o, h) and np.all(wd[1, 64:] > 0.4) and np.all(wd[1, :64] == 0)
