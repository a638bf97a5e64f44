"""Pins for the oracle's block glue (oracle/glue.py): closed-form values of SiLU,
its derivative checked by central finite differences of the forward (an independent
route to the same numbers), linearity in U, limits, and the gradient sum."""
import math

import numpy as np

import oracle


def test_silu_closed_forms():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    g = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -40.0, 800.0, -800.0])
    s = oracle.sigmoid(g)
    assert s[0] == 0.5 and abs(s[1] - 0.75) < 1e-15 and abs(s[2] - 0.25) < 1e-15
    assert s[3] == 1.0 - math.exp(-40.0) or abs(s[3] - 1.0) < 1e-17
    assert 0 < s[4] < 1e-17 and s[5] == 1.0 and s[6] == 0.0   # no overflow warnings either way
    h = oracle.silu_gate_fwd(g, np.ones_like(g))
    assert h[0] == 0.0
    assert abs(h[1] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(h[2] + 0.25 * math.log(3.0)) < 1e-15
    assert abs(h[3] - 40.0) < 1e-12 and abs(h[4]) < 1e-15 and h[5] == 800.0 and h[6] == 0.0
    # SiLU'(0) = 1/2; SiLU'(ln 3) = 3/4 (1 + ln3/4)
    dg, du = oracle.silu_gate_bwd(np.array([0.0, math.log(3.0)]), np.ones(2), np.ones(2))
    assert dg[0] == 0.5 and abs(dg[1] - 0.75 * (1 + math.log(3.0) / 4)) < 1e-15
    assert du[0] == 0.0 and abs(du[1] - 0.75 * math.log(3.0)) < 1e-15


def test_silu_gate_backward_by_finite_differences():
    rng = np.random.default_rng(3)
    g = rng.standard_normal(400) * 3.0
    g[:3] = [-1.2784645427610738, 0.0, 5.0]   # near the zero of SiLU', at 0, large
    u = rng.standard_normal(400)
    dh = rng.standard_normal(400)
    dg, du = oracle.silu_gate_bwd(g, u, dh)
    eps = 1e-6
    fd_g = (oracle.silu_gate_fwd(g + eps, u) - oracle.silu_gate_fwd(g - eps, u)) / (2 * eps) * dh
    fd_u = (oracle.silu_gate_fwd(g, u + eps) - oracle.silu_gate_fwd(g, u - eps)) / (2 * eps) * dh
    assert np.max(np.abs(dg - fd_g)) < 1e-8
    assert np.max(np.abs(du - fd_u)) < 1e-8


def test_silu_gate_linear_in_u_and_sign():
    rng = np.random.default_rng(4)
    g = rng.standard_normal(100)
    u = rng.standard_normal(100)
    h = oracle.silu_gate_fwd(g, u)
    assert np.allclose(oracle.silu_gate_fwd(g, 3.0 * u), 3.0 * h, rtol=1e-15, atol=0)
    # SiLU(g) has the sign of g, and |SiLU(g)| <= |g|
    s = oracle.silu_gate_fwd(g, np.ones_like(g))
    assert np.all(np.sign(s) == np.sign(g)) and np.all(np.abs(s) <= np.abs(g))


def test_grad_sum():
    a = np.array([[1.0, -2.0], [0.5, 0.0]])
    b = np.array([[0.25, 2.0], [-0.5, 3.0]])
    assert np.array_equal(oracle.grad_sum([a, b]), [[1.25, 0.0], [0.0, 3.0]])
    assert np.array_equal(oracle.grad_sum([a]), a)
