"""GPU parity of the codebook variants (INT4, FP4 and NF4 through the codebook
entry points; with and without double quantization) against oracle.codebooks:
bit-exact codes, block scales and float32 / bf16 reconstructions, values next
to every decision midpoint, the linear layer and the merge on a non-NF4
weight, and the reconstruction-MSE study ([TT] §5 "NF4"; [MC] "What the
experiments establish")."""
import numpy as np
import pytest
import torch

import oracle
from oracle import codebooks as cbk
from parity import assert_close, to_np
import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_fine_nf4_amd as nf4  # noqa: E402

DEV = "cuda:0"
F32 = np.float32
CB = list(cbk.CODEBOOKS)


def _weights(n, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(n) * 0.02).astype(F32)
    w[::53] *= 8.0
    return w


@pytest.mark.parametrize("cb", CB)
@pytest.mark.parametrize("n", [1, 63, 65, 513, 64 * 777 + 5, 1 << 20])
def test_quantize_and_dequantize(cb, n):
    print(f"codebook {cb} n={n}", flush=True)
    c = nf4.CODEBOOKS[cb]
    w = _weights(n, n + c)
    codes, absmax = nf4.qlora_quantize(torch.from_numpy(w).to(DEV), codebook=c)
    qa, s2, mean = nf4.qlora_double_quant(absmax)
    f32 = nf4.qlora_dequantize(codes, qa, s2, mean, n, torch.float32, codebook=c)
    b16 = nf4.qlora_dequantize(codes, qa, s2, mean, n, torch.bfloat16, codebook=c)
    nd = nf4.qlora_dequantize_nodq(codes, absmax, n, torch.float32, codebook=c)
    ndb = nf4.qlora_dequantize_nodq(codes, absmax, n, torch.bfloat16, codebook=c)
    torch.cuda.synchronize()
    rp, ra = cbk.quantize(w, cb)
    rq, rs2, rmean = oracle.double_quant(ra)
    assert np.array_equal(to_np(codes), rp)
    assert np.array_equal(to_np(absmax).view(np.uint32), ra.view(np.uint32))
    ref = cbk.dequantize(rp, rq, rs2, rmean, n, cb)
    assert np.array_equal(to_np(f32).view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(b16.cpu().view(torch.int16).numpy().view(np.uint16), oracle.f32_to_bf16_bits(ref))
    ref_nd = cbk.dequantize_no_dq(rp, ra, n, cb)
    assert np.array_equal(to_np(nd).view(np.uint32), ref_nd.view(np.uint32))
    assert np.array_equal(ndb.cpu().view(torch.int16).numpy().view(np.uint16), oracle.f32_to_bf16_bits(ref_nd))


@pytest.mark.parametrize("cb", CB)
def test_values_next_to_every_midpoint(cb):
    """Blocks whose absmax is 1 and whose other values sit one or two float32 steps
    either side of each midpoint: the encoder's guard band and exact fallback decide."""
    print(f"codebook {cb} midpoints", flush=True)
    mids = cbk.midpoints(cb)
    mids = mids[np.abs(mids) <= 1]
    vals = []
    for m in mids:
        f = F32(m)
        for k in (-2, -1, 0, 1, 2):
            x = f
            for _ in range(abs(k)):
                x = np.nextafter(x, F32(np.sign(k) * 2.0))
            vals.append(x)
    vals = np.array(vals, F32)
    nblk = (vals.size + 62) // 63
    w = np.zeros(nblk * 64, F32)
    for b in range(nblk):
        chunk = vals[63 * b:63 * (b + 1)]
        w[64 * b] = 1.0
        w[64 * b + 1:64 * b + 1 + chunk.size] = chunk
    codes, absmax = nf4.qlora_quantize(torch.from_numpy(w).to(DEV), codebook=nf4.CODEBOOKS[cb])
    torch.cuda.synchronize()
    rp, ra = cbk.quantize(w, cb)
    assert np.array_equal(to_np(codes), rp) and np.array_equal(to_np(absmax), ra)


@pytest.mark.parametrize("cb", ["int4", "fp4"])
def test_linear_layer_on_a_variant_weight(cb):
    M, h, o, r, s = 130, 512, 384, 16, 2.0
    print(f"linear {cb}", flush=True)
    w, l1, l2, x, dy = wl.small_linear(h, o, r, M, seed=77)
    W = nf4.quantize_weight(w.to(DEV), codebook=nf4.CODEBOOKS[cb])
    L1, L2, X, dY = l1.to(DEV), l2.to(DEV), x.to(DEV), dy.to(DEV)
    Y, T = nf4.qlora_linear_fwd(W, X, L1, L2, s)
    dX, dL1, dL2 = nf4.qlora_linear_bwd(W, X, T, dY, L1, L2, s)
    torch.cuda.synchronize()
    rp, ra = cbk.quantize(w.numpy().ravel(), cb)
    q, s2, mean = oracle.double_quant(ra)
    wh = cbk.dequantize(rp, q, s2, mean, h * o, cb).reshape(o, h)
    X64, DY64 = to_np(x).astype(np.float64), to_np(dy).astype(np.float64)
    rY, _ = oracle.linear_fwd(wh, X64, to_np(l1), to_np(l2), s)
    rdX, rdL1, rdL2 = oracle.linear_bwd(wh, X64, DY64, to_np(l1), to_np(l2), s)
    assert_close("Y", to_np(Y), rY)
    assert_close("dX", to_np(dX), rdX)
    assert_close("dL1", to_np(dL1), rdL1)
    assert_close("dL2", to_np(dL2), rdL2)


@pytest.mark.parametrize("cb", ["int4", "fp4"])
def test_merge_requantize_keeps_the_codebook(cb):
    h, o, r, s = 256, 192, 8, 1.0
    w, l1, l2, _, _ = wl.small_linear(h, o, r, 4, seed=5, lora_std=0.05)
    c = nf4.CODEBOOKS[cb]
    W = nf4.quantize_weight(w.to(DEV), codebook=c)
    L1, L2 = l1.to(DEV), l2.to(DEV)
    codes, absmax = nf4.qlora_merge_requantize(W, L1, L2, s)
    merged = nf4.qlora_merge_adapter(W, L1, L2, s, torch.float32)
    c2, a2 = nf4.qlora_quantize(merged, codebook=c)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(codes), to_np(c2))
    assert np.array_equal(to_np(absmax).view(np.uint32), to_np(a2).view(np.uint32))
    rp, ra = cbk.quantize(w.numpy().ravel(), cb)
    q, s2, mean = oracle.double_quant(ra)
    wh = cbk.dequantize(rp, q, s2, mean, h * o, cb)
    m0 = nf4.qlora_merge_adapter(W, None, None, s, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(m0).ravel().view(np.uint32), wh.view(np.uint32))


def test_reconstruction_mse_study_matches_the_oracle():
    """The study on 2^20 N(0, 1) weights: GPU reconstructions are bit-exact, so the MSE
    values equal the oracle's; NF4 has the lowest error."""
    n = 1 << 20
    w = np.random.default_rng(1).standard_normal(n).astype(F32)
    mse = {}
    for cb in CB:
        c = nf4.CODEBOOKS[cb]
        codes, absmax = nf4.qlora_quantize(torch.from_numpy(w).to(DEV), codebook=c)
        qa, s2, mean = nf4.qlora_double_quant(absmax)
        rec = nf4.qlora_dequantize(codes, qa, s2, mean, n, torch.float32, codebook=c)
        torch.cuda.synchronize()
        d = to_np(rec).astype(np.float64) - w
        mse[cb] = float(np.mean(d * d))
        assert mse[cb] == cbk.reconstruction_mse(w, cb, dq=True)
    print(f"  mse {mse}", flush=True)
    assert mse["nf4"] < min(mse["int4"], mse["fp4"])
