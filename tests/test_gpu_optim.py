"""GPU parity of qlora_adamw_step against the float64 oracle (AdamW on adapter
parameters; [TT] §4 "One QLoRA Training Step, End to End", [TT] §7 "Paged
Optimizers").

The kernel computes in float32 from float32 inputs.  One step's error bound,
from the float32 roundings of its operations (u = 2^-24): m within
em = 4u (|m| + |g|), v within 4u (v + g^2), and p within
4u |p| + 16u |upd| + 2 lr / (1 - b1^t) * em / den, where
upd = lr / (1 - b1^t) * m / den, den = sqrt(v) / sqrt(1 - b2^t) + eps, is the
oracle's update: the division, square root and host-rounded constants each
contribute a few u relative to upd, and the new m's own rounding error passes
through the division unchanged (it is not relative to the new m, which can be
small when b1 m and (1 - b1) g nearly cancel).  Over k steps the bounds add.
The entry point takes lr, beta1, beta2, eps and wd as float32, so the oracle
is evaluated at those float32 values (0.999f differs from 0.999 by 1.3e-5
relative in 1 - beta2)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_fine_nf4_amd as nf4  # noqa: E402

DEV = "cuda:0"
U = 2.0 ** -24


def _state(n, seed, steps_taken=0):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0, n)).astype(np.float32)
    if steps_taken:
        m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        v = ((rng.standard_normal(n) * 1e-2) ** 2).astype(np.float32)
    else:
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
    return p, g, m, v


def _run(p, g, m, v, t, hp, bf16=False, pinned=False):
    def place(a):
        x = torch.from_numpy(a.copy())
        return x.pin_memory() if pinned else x.to(DEV)
    P, G, M, V = (place(a) for a in (p, g, m, v))
    if pinned:
        P, G = torch.from_numpy(p.copy()).to(DEV), torch.from_numpy(g.copy()).to(DEV)
    B = torch.empty(p.size, dtype=torch.bfloat16, device=DEV) if bf16 else None
    nf4.qlora_adamw_step(P, G, M, V, t, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"], B)
    torch.cuda.synchronize()
    out = [x.cpu().numpy() for x in (P, M, V)]
    return out + ([B] if bf16 else [])


def _f32(hp):
    return {k: float(np.float32(x)) for k, x in hp.items()}


def _check_one_step(p, g, m, v, t, hp, got):
    hp = _f32(hp)
    rp, rm, rv = oracle.adamw_step(p, g, m, v, t, **hp)
    upd = np.abs(p.astype(np.float64) * (1 - hp["lr"] * hp["wd"]) - rp)
    gp, gm, gv = (x.astype(np.float64) for x in got[:3])
    p64, g64, m64, v64 = (x.astype(np.float64) for x in (p, g, m, v))
    em = 4 * U * (np.abs(m64) + np.abs(g64))
    assert np.all(np.abs(gm - rm) <= em + 1e-45)
    assert np.all(np.abs(gv - rv) <= 4 * U * (v64 + g64 * g64) + 1e-45)
    err = np.abs(gp - rp)
    den = np.sqrt(rv) / np.sqrt(1 - hp["beta2"] ** t) + hp["eps"]
    bound = 4 * U * np.abs(p64) + 16 * U * upd + 2 * hp["lr"] / (1 - hp["beta1"] ** t) * em / den + 1e-45
    print(f"  p: max err/bound = {np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound)


HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1000, 65537])
@pytest.mark.parametrize("t", [1, 7, 1000])
def test_adamw_one_step(n, t):
    print(f"adamw n={n} t={t}", flush=True)
    p, g, m, v = _state(n, seed=n + t, steps_taken=t - 1)
    _check_one_step(p, g, m, v, t, HP, _run(p, g, m, v, t, HP))


@pytest.mark.parametrize("hp", [dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-6, wd=0.0),
                                dict(lr=0.1, beta1=0.5, beta2=0.75, eps=1e-3, wd=0.5),
                                dict(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.1)])
def test_adamw_hyperparameter_edges(hp):
    print(f"adamw hp={hp}", flush=True)
    p, g, m, v = _state(777, seed=3, steps_taken=4)
    _check_one_step(p, g, m, v, 5, hp, _run(p, g, m, v, 5, hp))


def test_adamw_bf16_copy_is_rne_of_the_float32_result():
    p, g, m, v = _state(4099, seed=9)
    P, M, V, B = _run(p, g, m, v, 1, HP, bf16=True)
    ref = torch.from_numpy(P).to(torch.bfloat16)
    assert torch.equal(B.cpu().view(torch.int16), ref.view(torch.int16))


def test_adamw_twenty_steps():
    n = 5000
    p, _, m, v = _state(n, seed=11)
    rng = np.random.default_rng(12)
    P, M, V = (torch.from_numpy(a.copy()).to(DEV) for a in (p, m, v))
    rp, rm, rv = p.astype(np.float64), m.astype(np.float64), v.astype(np.float64)
    bound = np.zeros(n)
    for t in range(1, 21):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0, n)).astype(np.float32)
        nf4.qlora_adamw_step(P, torch.from_numpy(g).to(DEV), M, V, t, **{k: HP[k] for k in ("lr", "beta1", "beta2", "eps")},
                             weight_decay=HP["wd"])
        prev, prevm = rp, rm
        rp, rm, rv = oracle.adamw_step(rp, g, rm, rv, t, **_f32(HP))
        den = np.sqrt(rv) / np.sqrt(1 - HP["beta2"] ** t) + HP["eps"]
        em = 8 * U * (np.abs(prevm) + np.abs(g))
        bound += (4 * U * np.abs(prev) + 32 * U * np.abs(prev * (1 - HP["lr"] * HP["wd"]) - rp)
                  + 2 * HP["lr"] / (1 - HP["beta1"] ** t) * em / den)
    torch.cuda.synchronize()
    err = np.abs(P.cpu().numpy().astype(np.float64) - rp)
    print(f"  20 steps: max err/bound = {np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound)


def test_adamw_state_in_pinned_host_memory_matches_device_state():
    p, g, m, v = _state(100003, seed=21, steps_taken=2)
    dev = _run(p, g, m, v, 3, HP)
    host = _run(p, g, m, v, 3, HP, pinned=True)
    for a, b in zip(dev, host):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_adamw_adapter_shapes_of_a_65b_projection():
    """L1 (8192 x 64) and L2 (64 x 8192) of one LLaMA-65B projection, flat: 1,048,576 values."""
    n = 2 * 8192 * 64
    p, g, m, v = _state(n, seed=31, steps_taken=9)
    _check_one_step(p, g, m, v, 10, HP, _run(p, g, m, v, 10, HP))
