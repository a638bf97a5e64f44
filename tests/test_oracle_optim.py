"""Pins of the oracle's adapter AdamW step against what fixes it independently:
PyTorch's own AdamW (a library routine, float64 on the CPU), the closed form of
the first step, and pure weight decay."""
import numpy as np
import pytest
import torch

import oracle

HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)


@pytest.mark.parametrize("seed", [0, 1])
def test_matches_torch_adamw_over_several_steps(seed):
    rng = np.random.default_rng(seed)
    n = 257
    p0 = rng.standard_normal(n) * 0.02
    grads = [rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0) for _ in range(6)]
    tp = torch.tensor(p0.copy(), dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["wd"], foreach=False, fused=False)
    p, m, v = p0, np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = oracle.adamw_step(p, g, m, v, t, **HP)
        st = opt.state[tp]
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-18)
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-20)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-30)


def test_first_step_moves_each_parameter_by_lr_against_the_gradient_sign():
    g = np.array([3.0, -2.0, 1e-3, -5e-2])
    p0 = np.array([0.5, -0.5, 0.25, 0.0])
    p, m, v = oracle.adamw_step(p0, g, np.zeros(4), np.zeros(4), 1, 1e-3, 0.9, 0.999, 0.0, 0.0)
    np.testing.assert_allclose(p, p0 - 1e-3 * np.sign(g), rtol=0, atol=1e-15)
    np.testing.assert_allclose(m, 0.1 * g)
    np.testing.assert_allclose(v, 0.001 * g * g)


def test_zero_gradient_is_pure_decay():
    p0 = np.array([1.0, -2.0, 3.0])
    m0 = np.array([0.1, 0.2, -0.3])
    v0 = np.array([0.0, 0.0, 0.0])
    p, m, v = oracle.adamw_step(p0, np.zeros(3), m0, v0, 5, 0.1, 0.5, 0.75, 1.0, 0.2)
    # v stays 0, so the update is lr / (1 - 0.5^5) * m / eps with m = 0.5 m0
    np.testing.assert_allclose(m, 0.5 * m0)
    np.testing.assert_allclose(v, v0)
    np.testing.assert_allclose(p, p0 * (1 - 0.1 * 0.2) - 0.1 / (1 - 0.5 ** 5) * (0.5 * m0) / 1.0)


def test_step_count_starts_at_one():
    with pytest.raises(ValueError):
        oracle.adamw_step(np.zeros(2), np.zeros(2), np.zeros(2), np.zeros(2), 0, **HP)
