"""GPU parity of qlora_linear_fwd / qlora_linear_bwd against the float64 oracle:
relative Frobenius error <= 1e-2 and max-abs error <= 2e-2 * max|ref| for Y, T,
dX, dL1, dL2.  Small shapes span several tiles with ragged token counts; the
workload shapes run at full size, compared in full where the oracle is quick
and on sampled token rows otherwise (dL1 and dL2 are always compared in full)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import assert_close, oracle_weight, to_np

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_fine_nf4_amd as nf4  # noqa: E402

DEV = "cuda:0"


def gpu_run(w, l1, l2, x, dy, s):
    W = nf4.quantize_weight(w.to(DEV))
    X, dY = x.to(DEV), dy.to(DEV)
    L1 = None if l1 is None else l1.to(DEV)
    L2 = None if l2 is None else l2.to(DEV)
    Y, T = nf4.qlora_linear_fwd(W, X, L1, L2, s)
    dX, dL1, dL2 = nf4.qlora_linear_bwd(W, X, T, dY, L1, L2, s)
    torch.cuda.synchronize()
    return Y, T, dX, dL1, dL2


def check_full(w, l1, l2, x, dy, s, label):
    print(f"linear {label}", flush=True)
    Y, T, dX, dL1, dL2 = gpu_run(w, l1, l2, x, dy, s)
    wh = oracle_weight(w)
    X, DY = to_np(x).astype(np.float64), to_np(dy).astype(np.float64)
    L1 = None if l1 is None else to_np(l1)
    L2 = None if l2 is None else to_np(l2)
    rY, rT = oracle.linear_fwd(wh, X, L1, L2, s)
    rdX, rdL1, rdL2 = oracle.linear_bwd(wh, X, DY, L1, L2, s)
    assert_close("Y", to_np(Y), rY)
    assert_close("dX", to_np(dX), rdX)
    if l1 is not None:
        assert_close("T", to_np(T), rT)
        assert_close("dL1", to_np(dL1), rdL1)
        assert_close("dL2", to_np(dL2), rdL2)


SMALL = [  # (M, h, o, r, s)
    (1, 64, 64, 0, 1.0),
    (3, 128, 192, 8, 2.0),
    (7, 320, 128, 4, 1.0),
    (12, 576, 192, 0, 1.0),
    (16, 1024, 1024, 8, 2.0),
    (17, 256, 320, 16, 2.0),
    (130, 512, 384, 5, 0.5),
    (300, 1024, 512, 64, 0.25),
    (513, 320, 640, 128, 1.5),
    (257, 576, 1088, 16, 2.0),
    (2050, 256, 320, 3, 1.0),     # rank-r products: 8 rows per workgroup, ragged last workgroup
    (4100, 192, 256, 100, 0.5),   # 16 rows per workgroup, ragged, r not a multiple of 8
]


@pytest.mark.parametrize("M,h,o,r,s", SMALL)
def test_linear_small(M, h, o, r, s):
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=M + h + o + r)
    check_full(w, l1, l2, x, dy, s, f"M={M} h={h} o={o} r={r}")


def test_linear_zero_weight_isolates_adapter():
    M, h, o, r, s = 96, 256, 192, 16, 2.0
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=5, lora_std=0.05)
    check_full(torch.zeros_like(w), l1, l2, x, dy, s, "W=0")


def test_linear_workload_c1():
    c = wl.C1
    ls = c.linears[0]
    w = wl.base_weight(c, 0)
    l1, l2 = wl.lora_factors(c, 0)
    check_full(w, l1, l2, wl.activations(c, 0), wl.activations(c, 0, tensor=wl.TENSOR_DY), ls.s, c.name)


def test_linear_workload_c2():
    c = wl.C2
    ls = c.linears[0]
    w = wl.base_weight(c, 0)
    l1, l2 = wl.lora_factors(c, 0)
    check_full(w, l1, l2, wl.activations(c, 0), wl.activations(c, 0, tensor=wl.TENSOR_DY), ls.s, c.name)


def check_sampled(c, li, nrows=48):
    """Full-size linear of a workload: Y and dX on sampled token rows, T/dL1/dL2 in full."""
    ls = c.linears[li]
    print(f"linear {c.name}/{ls.name} sampled", flush=True)
    w = wl.base_weight(c, li)
    l1, l2 = wl.lora_factors(c, li)
    x = wl.activations(c, li)
    dy = wl.activations(c, li, tensor=wl.TENSOR_DY)
    Y, T, dX, dL1, dL2 = gpu_run(w, l1, l2, x, dy, ls.s)
    wh = oracle_weight(w)
    del w
    rows = np.unique(np.concatenate([np.random.default_rng(li).integers(0, c.tokens, nrows), [0, c.tokens - 1]]))
    X, DY = to_np(x).astype(np.float64), to_np(dy).astype(np.float64)
    L1, L2 = to_np(l1), to_np(l2)
    rY, rT = oracle.linear_fwd(wh, X[rows], L1, L2, ls.s)
    rdX, _, _ = oracle.linear_bwd(wh, X[rows], DY[rows], L1, L2, ls.s)
    assert_close("Y[rows]", to_np(Y)[rows], rY)
    assert_close("dX[rows]", to_np(dX)[rows], rdX)
    T64 = X @ L1.astype(np.float64)
    U64 = DY @ L2.astype(np.float64).T
    assert_close("T", to_np(T), T64)
    assert_close("dL1", to_np(dL1), ls.s * (X.T @ U64))
    assert_close("dL2", to_np(dL2), ls.s * (T64.T @ DY))


@pytest.mark.parametrize("li", [0, 2])
def test_linear_workload_c3_sampled(li):
    check_sampled(wl.C3, li)


@pytest.mark.parametrize("li", [0, 4, 6])
def test_linear_workload_c5_sampled(li):
    check_sampled(wl.C5, li)


@pytest.mark.parametrize("m", wl.C4_GEMV_TOKENS)
def test_gemv_workload_c4(m):
    c = wl.C4_GEMV
    print(f"gemv M={m}", flush=True)
    w = wl.base_weight(c, 0)
    x = wl.activations(c, 0, tokens=m)
    W = nf4.quantize_weight(w.to(DEV))
    Y, _ = nf4.qlora_linear_fwd(W, x.to(DEV), None, None, 1.0)
    torch.cuda.synchronize()
    wh = oracle_weight(w)
    rY, _ = oracle.linear_fwd(wh, to_np(x).astype(np.float64), None, None, 1.0)
    assert_close("Y", to_np(Y), rY)


def test_adjoint_identities_on_gpu_outputs():
    """<dX, X> = <dY, Y> and <dL1, L1> = <dL2, L2> = <dY, Y - X W_hat> hold for the GPU
    outputs up to bf16 rounding (no oracle involved)."""
    c = wl.C2
    ls = c.linears[0]
    w = wl.base_weight(c, 0)
    l1, l2 = wl.lora_factors(c, 0)
    x, dy = wl.activations(c, 0), wl.activations(c, 0, tensor=wl.TENSOR_DY)
    Y, T, dX, dL1, dL2 = gpu_run(w, l1, l2, x, dy, ls.s)
    W = nf4.quantize_weight(w.to(DEV))
    Yb, _ = nf4.qlora_linear_fwd(W, x.to(DEV), None, None, 1.0)
    torch.cuda.synchronize()
    f = lambda a: to_np(a).astype(np.float64)
    lhs = np.sum(f(dX) * f(x))
    rhs = np.sum(f(dy) * f(Y))
    assert abs(lhs - rhs) <= 2e-2 * np.sqrt(np.sum(f(dX) ** 2) * np.sum(f(x) ** 2))
    a1 = np.sum(f(dL1) * f(l1))
    a2 = np.sum(f(dL2) * f(l2))
    lora = np.sum(f(dy) * (f(Y) - f(Yb)))
    scale = np.sqrt(np.sum(f(dL2) ** 2) * np.sum(f(l2) ** 2))
    assert abs(a1 - a2) <= 2e-2 * scale and abs(a1 - lora) <= 5e-2 * scale


FEW_TOKEN_BWD = [  # (M, h, o, r, s): the few-token backward (dX GEMV), several column tiles and row chunks
    (1, 8192, 4096, 0, 1.0),
    (2, 4096, 11008, 64, 0.25),
    (4, 1536, 2048, 8, 2.0),
    (9, 11008, 4096, 16, 2.0),
    (16, 2560, 1088, 128, 0.5),
]


@pytest.mark.parametrize("M,h,o,r,s", FEW_TOKEN_BWD)
def test_few_token_backward(M, h, o, r, s):
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=3 * M + h + r)
    check_full(w, l1, l2, x, dy, s, f"few-token M={M} h={h} o={o} r={r}")
