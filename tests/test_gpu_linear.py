"""GPU parity of qlora_linear_fwd / qlora_linear_bwd against the float64 oracle:
relative Frobenius error <= 1e-2 and max-abs error <= 2e-2 * max|ref| for Y, T,
dX, dL1, dL2, every output compared in full against oracle.linear_fwd /
oracle.linear_bwd.  Small shapes span several tiles with ragged token counts; the
workload shapes run at full size.  The rank-r term is isolated on each fused-GEMM
tile size (W = 0, and adapters large enough to be 25-70 % of the output, with one
and two rank-r K steps), since with the workloads' own small adapters it is about
1 % of Y and dX and a 1e-2 check could not see it."""
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
    (33000, 128, 192, 8, 1.0),    # rank-r products in one K range (no split partials), ragged rows
    (32769, 64, 128, 100, 0.5),   # the same with r not a multiple of 8 (element-wise L1 copies)
    (64, 8192, 8192, 16, 2.0),    # r <= 16 adapter gradients on 64-wide tiles (256 of them)
    (40, 8192, 8448, 5, 1.0),     # the same with r not a multiple of 8, ragged token slab
    (200, 512, 768, 40, 1.0),     # split adapter gradients and rank products with 48 rank columns
    (150, 640, 384, 27, 0.5),     # 32 rank columns, r not a multiple of 8
    (96, 8192, 8192, 64, 0.25),   # 64 rank columns, 256 gradient tiles
    (130, 512, 384, 13, 1.0),     # one pass, r not a multiple of 8: element-wise Q copies
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


def check_workload(c, li):
    """Full-size linear of a workload, every output compared in full."""
    ls = c.linears[li]
    w = wl.base_weight(c, li)
    l1, l2 = wl.lora_factors(c, li)
    x = wl.activations(c, li)
    dy = wl.activations(c, li, tensor=wl.TENSOR_DY)
    check_full(w, l1, l2, x, dy, ls.s, f"{c.name}/{ls.name}")


def test_linear_256x128_tiles_ragged():
    """M = 2000, h = o = 2624 selects the 256x128 fused-GEMM tiles in both
    directions, with partial last tiles along M (208 rows) and N (64 columns);
    compared in full."""
    M, h, o, r, s = 2000, 2624, 2624, 16, 2.0
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=2000)
    check_full(w, l1, l2, x, dy, s, f"M={M} h={h} o={o} r={r} (256x128 tiles)")


def test_linear_256x256_tiles_ragged():
    """M = 3000, h = o = 5184 selects the 256x256 fused-GEMM tiles in both
    directions, with partial last tiles along M (184 rows) and N (64 columns)."""
    M, h, o, r, s = 3000, 5184, 5184, 16, 0.5
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=3000)
    check_full(w, l1, l2, x, dy, s, f"M={M} h={h} o={o} r={r} (256x256 tiles)")


# The rank-r K steps of each fused-GEMM tile size, isolated.  (M, h, o) picks the
# tile: 4096 x 4096 x 4096 and 3000 x 5184 x 5184 the 256x256 tiles, 2000 x 2624 x 2624
# the 256x128 tiles (both directions).  r = 100 and 128 take two rank-r K steps.
@pytest.mark.parametrize("r,s", [(16, 2.0), (64, 0.25), (128, 0.5)])
def test_rank_r_only_256x256_tiles(r, s):
    """W = 0: Y = s X L1 L2 and dX = s dY L2^T L1^T come from the rank-r steps alone."""
    M, h, o = 4096, 4096, 4096
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=40 + r, lora_std=0.05)
    check_full(torch.zeros_like(w), l1, l2, x, dy, s, f"W=0 M={M} h={h} o={o} r={r} (256x256 tiles)")


@pytest.mark.parametrize("M,h,o,r,s", [(2000, 2624, 2624, 100, 0.5), (2000, 2624, 2624, 128, 0.5),
                                       (3000, 5184, 5184, 100, 0.5), (3000, 5184, 5184, 128, 0.25)])
def test_large_adapter_wide_tiles(M, h, o, r, s):
    """Adapters with std 0.05: the rank-r term is 25-70 % of Y and dX, so a dropped or
    mis-scaled K step fails the 1e-2 check."""
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=M + r, lora_std=0.05)
    check_full(w, l1, l2, x, dy, s, f"M={M} h={h} o={o} r={r} lora_std=0.05")


def test_large_adapter_c5_shape():
    """The 65B block's attention projection shape (2048 x 8192 x 8192, r = 64, s = 0.25,
    256x256 tiles) with adapters of std 0.05: the rank-r term is about 25 % of Y."""
    M, h, o, r, s = 2048, 8192, 8192, 64, 0.25
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=65, lora_std=0.05)
    check_full(w, l1, l2, x, dy, s, f"C5 shape M={M} h={h} o={o} r={r} lora_std=0.05")


@pytest.mark.parametrize("li", [0, 2])
def test_linear_workload_c3(li):
    check_workload(wl.C3, li)


@pytest.mark.parametrize("li", [0, 4, 6])
def test_linear_workload_c5(li):
    check_workload(wl.C5, li)


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


FEW_TOKEN_FWD = [  # (M, h, o, r, s): the few-token forward with K not a whole number of 16-block
    # prefetch rounds or of 256-weight activation phases, one or many workgroups, every token class
    (1, 2368, 640, 8, 1.0),
    (2, 64, 4096, 16, 2.0),
    (4, 4160, 64, 0, 1.0),
    (5, 192, 1152, 4, 0.5),
    (13, 1088, 320, 32, 2.0),
    (16, 5184, 192, 0, 1.0),
    (1, 11008, 256, 16, 2.0),     # one token, K above 8192: eight 1 KB loads per row
    (1, 16384, 128, 0, 1.0),
    (1, 16448, 64, 8, 0.5),       # one token, K above 16384: the MFMA kernel
    (1, 64, 131136, 4, 1.0),      # one token, 65 rows per wave: results flushed every 64 rows
]


@pytest.mark.parametrize("M,h,o,r,s", FEW_TOKEN_FWD)
def test_few_token_forward(M, h, o, r, s):
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=5 * M + h + o + r)
    check_full(w, l1, l2, x, dy, s, f"few-token fwd M={M} h={h} o={o} r={r}")


@pytest.mark.parametrize("M,h,o,r,s", FEW_TOKEN_BWD)
def test_few_token_backward(M, h, o, r, s):
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=3 * M + h + r)
    check_full(w, l1, l2, x, dy, s, f"few-token M={M} h={h} o={o} r={r}")


class _HipEvents:
    """Raw hipEvent_t handles (the library records them; torch would refuse to time
    events it did not record itself)."""

    def __init__(self):
        import ctypes
        import os
        path = None
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
        self.ct = ctypes
        self.hip = ctypes.CDLL(path or os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.live = []

    def create(self):
        ev = self.ct.c_void_p()
        assert self.hip.hipEventCreate(self.ct.byref(ev)) == 0
        self.live.append(ev)
        return ev

    def elapsed(self, a, b):
        """(status, ms): status is non-zero when either event was never recorded (the
        runtime's last-error state is cleared then, so no later launch check sees it)."""
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            self.hip.hipGetLastError()
        return rc, ms.value

    def close(self):
        for ev in self.live:
            self.hip.hipEventDestroy(ev)


@pytest.mark.parametrize("M,expect", [(512, (0, 1)), (4, (1, 2))])
def test_timing_hook_slots(M, expect):
    """qlora_set_timing_events: slot 0 brackets the forward fused GEMM, slot 1 the
    dX kernel (the fused GEMM, or for M <= 16 the few-token dX kernel), slot 2 the
    few-token forward.  A slot whose kernel does not run leaves its events
    unrecorded, and NULL/NULL switches the hook off."""
    h, o, r, s = 512, 768, 8, 2.0
    print(f"timing hook M={M}", flush=True)
    g = torch.Generator().manual_seed(11)
    w = torch.randn(o, h, generator=g) * 0.02
    l1, l2 = torch.randn(h, r, generator=g) * 0.01, torch.randn(r, o, generator=g) * 0.01
    x = torch.randn(M, h, generator=g).to(torch.bfloat16)
    dy = torch.randn(M, o, generator=g).to(torch.bfloat16)
    W = nf4.quantize_weight(w.to(DEV))
    X, dY, L1, L2 = x.to(DEV), dy.to(DEV), l1.to(DEV).to(torch.bfloat16), l2.to(DEV).to(torch.bfloat16)
    hev = _HipEvents()
    slots = [nf4.TIMED_GEMM_FWD, nf4.TIMED_GEMM_DX, nf4.TIMED_GEMV]
    evs = {k: (hev.create(), hev.create()) for k in slots}
    try:
        for k in slots:
            nf4.qlora_set_timing_events(k, *evs[k])
        Y, T = nf4.qlora_linear_fwd(W, X, L1, L2, s)
        nf4.qlora_linear_bwd(W, X, T, dY, L1, L2, s)
        torch.cuda.synchronize()
    finally:
        for k in slots:
            nf4.qlora_set_timing_events(k, None, None)
    first = {}
    for k in slots:
        rc, ms = hev.elapsed(*evs[k])
        if k in expect:
            assert rc == 0 and 0.0 < ms < 1000.0, (k, rc, ms)
            first[k] = ms
        else:
            assert rc != 0, f"slot {k} recorded although its kernel did not run"
    # switched off: another pass records nothing, so the timed pairs keep their values
    Y, T = nf4.qlora_linear_fwd(W, X, L1, L2, s)
    nf4.qlora_linear_bwd(W, X, T, dY, L1, L2, s)
    torch.cuda.synchronize()
    for k in expect:
        assert hev.elapsed(*evs[k]) == (0, first[k])
    hev.close()


def test_few_token_backward_many_gradient_tiles():
    """M = 1 with h + o > 131072 (h = 128, o = 131072, r = 8): the adapter gradients have
    1025 tiles, more than the one 1024-thread workgroup of the rank-r launch that clears
    their split counters.  The workspace starts as garbage and is reused by a second call
    (which then finds the first call's counts), and both calls must match the oracle."""
    M, h, o, r, s = 1, 128, 131072, 8, 2.0
    print(f"few-token bwd M={M} h={h} o={o} r={r} (1025 gradient tiles)", flush=True)
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=131, lora_std=0.05)
    W = nf4.quantize_weight(w.to(DEV))
    X, dY, L1, L2 = x.to(DEV), dy.to(DEV), l1.to(DEV), l2.to(DEV)
    Y, T = nf4.qlora_linear_fwd(W, X, L1, L2, s)
    ws = torch.full((nf4.workspace_size(nf4.QLORA_OP_LINEAR_BWD, M, h, o, r),), 0x7F, dtype=torch.uint8,
                    device=DEV)
    wh = oracle_weight(w)
    rdX, rdL1, rdL2 = oracle.linear_bwd(wh, to_np(x).astype(np.float64), to_np(dy).astype(np.float64),
                                        to_np(l1), to_np(l2), s)
    for call in range(2):
        dX, dL1, dL2 = nf4.qlora_linear_bwd(W, X, T, dY, L1, L2, s, workspace=ws)
        torch.cuda.synchronize()
        print(f" call {call}", flush=True)
        assert_close("dX", to_np(dX), rdX)
        assert_close("dL1", to_np(dL1), rdL1)
        assert_close("dL2", to_np(dL2), rdL2)
