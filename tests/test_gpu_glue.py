"""GPU parity of the block glue (qlora_silu_gate_fwd / _bwd, qlora_grad_sum) against
the float64 oracle (oracle/glue.py).

Per-element bound: the float32 arithmetic then one round to nearest even in bf16,
whose half-ulp is at most 2^-8 of the value, so |got - ref| <= 2^-8 |ref| + e.  e
covers float32 error: exp's relative error grows with |g| (about |g| 2^-24), the
factor 1 + g(1 - sigmoid(g)) of dG cancels near g = -1.28, so e scales with the
operand magnitudes: 2^-14 |g u| for H, 2^-14 |dh g| for dU, 2^-14 |dh u| (1 + |g|)
for dG, and (k + 1) 2^-24 sum|x| for a sum of k terms.  Sizes cover the 8-wide vector
path, its scalar tail and the C3 / C5 feed-forward shapes."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import REL_FROB_TOL

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_fine_nf4_amd as nf4  # noqa: E402

DEV = "cuda:0"


def bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def f64(t):
    return t.detach().cpu().float().numpy().astype(np.float64)


def within(name, got, ref, slack):
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + slack
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, (name, bad[:5], got.ravel()[bad[:5]], ref.ravel()[bad[:5]])
    den = np.linalg.norm(ref)
    if den > 0:
        assert np.linalg.norm(got - ref) / den <= REL_FROB_TOL


def special_gates(n, rng):
    g = rng.standard_normal(n) * 3.0
    sp = [0.0, -0.0, 1e-30, -1e-30, 88.0, -88.0, 100.0, -100.0, 1e30, -1e30, -1.2784645, -1.28, -1.27, 0.5]
    k = min(n, len(sp))
    g[:k] = sp[:k]
    return g


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 65536 + 3, 4096 * 11008])
def test_silu_gate_parity(n):
    print(f"silu gate n={n}", flush=True)
    rng = np.random.default_rng(n)
    G, U, dH = bf16(special_gates(n, rng)), bf16(rng.standard_normal(n)), bf16(rng.standard_normal(n))
    g, u, dh = f64(G), f64(U), f64(dH)
    H = nf4.qlora_silu_gate_fwd(G.to(DEV), U.to(DEV))
    dG, dU = nf4.qlora_silu_gate_bwd(G.to(DEV), U.to(DEV), dH.to(DEV))
    torch.cuda.synchronize()
    rH = oracle.silu_gate_fwd(g, u)
    rdG, rdU = oracle.silu_gate_bwd(g, u, dh)
    within("H", f64(H), rH, 2.0 ** -14 * np.abs(g * u))
    within("dU", f64(dU), rdU, 2.0 ** -14 * np.abs(dh * g))
    within("dG", f64(dG), rdG, 2.0 ** -14 * np.abs(dh * u) * (1 + np.abs(g)))


def test_silu_gate_workload_shapes():
    """The C5 feed-forward shape (2048 tokens x 22016) with the workload's seeded
    N(0, 1) activations."""
    c = wl.C5
    G = wl.activations(c, 4, width=22016, tensor=wl.TENSOR_AUX)
    U = wl.activations(c, 5, width=22016, tensor=wl.TENSOR_AUX)
    dH = wl.activations(c, 6, width=22016, tensor=wl.TENSOR_DY)
    print("silu gate C5 shape", flush=True)
    H = nf4.qlora_silu_gate_fwd(G.to(DEV), U.to(DEV))
    dG, dU = nf4.qlora_silu_gate_bwd(G.to(DEV), U.to(DEV), dH.to(DEV))
    torch.cuda.synchronize()
    g, u, dh = f64(G), f64(U), f64(dH)
    within("H", f64(H), oracle.silu_gate_fwd(g, u), 2.0 ** -14 * np.abs(g * u))
    rdG, rdU = oracle.silu_gate_bwd(g, u, dh)
    within("dU", f64(dU), rdU, 2.0 ** -14 * np.abs(dh * g))
    within("dG", f64(dG), rdG, 2.0 ** -14 * np.abs(dh * u) * (1 + np.abs(g)))


@pytest.mark.parametrize("k,n", [(1, 5), (2, 8), (5, 1000003), (8, 4096)])
def test_grad_sum_parity(k, n):
    print(f"grad sum k={k} n={n}", flush=True)
    rng = np.random.default_rng(k * n)
    parts = [bf16(rng.standard_normal(n) * 10.0 ** rng.integers(-3, 3)) for _ in range(k)]
    dev = [p.to(DEV) for p in parts]
    out = nf4.qlora_grad_sum(dev)
    torch.cuda.synchronize()
    ref = oracle.grad_sum([f64(p) for p in parts])
    mag = sum(np.abs(f64(p)) for p in parts)
    within("sum", f64(out), ref, (k + 1) * 2.0 ** -24 * mag)
    # in place: the result replaces the first part
    nf4.qlora_grad_sum(dev, out=dev[0])
    torch.cuda.synchronize()
    within("sum in place", f64(dev[0]), ref, (k + 1) * 2.0 ** -24 * mag)
