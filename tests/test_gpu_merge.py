"""GPU parity of qlora_merge_adapter / qlora_merge_requantize against the oracle's
merged weight ([TT] §11 "Saving, Loading, and Merging QLoRA Adapters").

The merged weight is W_hat + s * P with P = L1 L2 summed in float32 in an order
the kernel chooses (MFMA accumulation), so the float32 output is compared with
the oracle's float32 merge element by element within a summation bound:
r terms summed in any order, then one rounding of s * P and one of the final
add, each at most u = 2^-24 relative to the magnitude |w_hat| + |s| sum|L1||L2|;
the bound is doubled because the matrix cores' internal accumulation rounding
is not specified as round-to-nearest.  Without an adapter (r = 0) and with
s = 0 the merge is exact, and the comparison is bit for bit.

Re-quantization is an integer decision on a float32 value, so the kernel's codes
are compared bit for bit with qlora_quantize run on the kernel's own float32
merge (two entry points, one decision), and with the oracle's quantization of
the oracle's merge wherever the oracle's normalised value is farther from a
level midpoint than the summation bound can move it; elsewhere the two codes
must be neighbouring levels."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import to_np

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_fine_nf4_amd as nf4  # noqa: E402

DEV = "cuda:0"
U = 2.0 ** -24


def _problem(h, o, r, seed, lora_std=0.02):
    w, l1, l2, _, _ = wl.small_linear(h, o, r, 4, seed=seed, lora_std=lora_std)
    p, a = oracle.quantize(w.numpy().ravel())
    q, s2, mean = oracle.double_quant(a)
    L1 = None if l1 is None else l1.float().numpy()
    L2 = None if l2 is None else l2.float().numpy()
    W = nf4.quantize_weight(w.to(DEV))
    # the GPU weight is the oracle's, bit for bit (the codec parity tests pin this)
    assert np.array_equal(to_np(W.codes), p) and np.array_equal(to_np(W.qabsmax), q)
    assert np.array_equal(to_np(W.scale2), s2) and to_np(W.mean)[0] == mean
    gl1 = None if l1 is None else l1.to(DEV)
    gl2 = None if l2 is None else l2.to(DEV)
    return W, gl1, gl2, (p, q, s2, mean, L1, L2)


def _bound(ref_parts, h, o, s):
    p, q, s2, mean, L1, L2 = ref_parts
    wh = oracle.dequantized_weight(p, q, s2, mean, h, o).astype(np.float64)
    if L1 is None:
        return np.zeros_like(wh)
    r = L1.shape[1]
    mag = np.abs(wh) + abs(s) * (np.abs(L1.astype(np.float64)) @ np.abs(L2.astype(np.float64))).T
    return 2.0 * (r + 3) * U * mag


def _rne_bf16(x32: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(x32))


SHAPES = [  # (h, o, r, s)
    (64, 64, 1, 2.0),
    (128, 192, 8, 0.5),
    (320, 128, 16, 2.0),
    (576, 320, 32, 1.5),
    (1024, 512, 64, 0.25),
    (256, 640, 100, 1.0),
    (512, 256, 128, 2.0),
]


@pytest.mark.parametrize("h,o,r,s", SHAPES)
def test_merge_f32_and_bf16(h, o, r, s):
    print(f"merge h={h} o={o} r={r} s={s}", flush=True)
    W, L1, L2, parts = _problem(h, o, r, seed=h + o + r)
    got = nf4.qlora_merge_adapter(W, L1, L2, s, torch.float32)
    gb = nf4.qlora_merge_adapter(W, L1, L2, s, torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.merged_weight(*parts[:4], h, o, parts[4], parts[5], s)
    g = to_np(got).astype(np.float64)
    err = np.abs(g - ref.astype(np.float64))
    bound = _bound(parts, h, o, s)
    print(f"  max err/bound = {np.max(err / np.maximum(bound, 1e-45)):.3f}", flush=True)
    assert np.all(err <= bound)
    # the adapter term is large against the bound: a dropped or transposed term fails
    assert np.max(np.abs(ref - oracle.dequantized_weight(*parts[:4], h, o))) > 1e3 * np.max(bound)
    # bf16 output: round to nearest even of the float32 merge
    assert np.array_equal(to_np(gb).view(np.uint32), _rne_bf16(to_np(got)).view(np.uint32))


@pytest.mark.parametrize("h,o,r,s", [(128, 192, 8, 0.5), (576, 320, 32, 1.5), (512, 256, 128, 2.0),
                                     (1024, 512, 64, 3.0)])
def test_merge_requantize(h, o, r, s):
    print(f"merge_requantize h={h} o={o} r={r} s={s}", flush=True)
    W, L1, L2, parts = _problem(h, o, r, seed=7 * h + o + r, lora_std=0.05)
    codes, absmax = nf4.qlora_merge_requantize(W, L1, L2, s)
    merged = nf4.qlora_merge_adapter(W, L1, L2, s, torch.float32)
    c2, a2 = nf4.qlora_quantize(merged)
    torch.cuda.synchronize()
    gc, ga = to_np(codes), to_np(absmax)
    # one decision, two entry points: bit-exact
    assert np.array_equal(gc, to_np(c2))
    assert np.array_equal(ga.view(np.uint32), to_np(a2).view(np.uint32))
    # against the oracle's own merge and quantization
    ref = oracle.merged_weight(*parts[:4], h, o, parts[4], parts[5], s)
    pc, pa = oracle.quantize(ref.ravel())
    bound = _bound(parts, h, o, s).ravel()
    bmax = bound.reshape(-1, 64).max(axis=1)
    assert np.all(np.abs(ga.astype(np.float64) - pa) <= bmax)
    n = h * o
    gcode = oracle.unpack_codes(gc, n).astype(np.int64)
    rcode = oracle.unpack_codes(pc, n).astype(np.int64)
    x = (ref.ravel().astype(np.float64) / np.repeat(np.where(pa > 0, pa, 1.0), 64))
    mids = oracle.nf4_midpoints()
    dist = np.min(np.abs(x[:, None] - mids[None, :]), axis=1)
    # the normalised value can move by the merge bound plus the scale's own change, relative to the scale
    slack = 4.0 * (bound + np.repeat(bmax, 64)) / np.repeat(np.where(pa > 0, pa, 1.0), 64) + 4 * U
    firm = dist > slack
    mism = gcode != rcode
    print(f"  code mismatches {int(mism.sum())} of {n} ({int((~firm).sum())} near a midpoint)", flush=True)
    assert not np.any(mism & firm)
    assert np.all(np.abs(gcode - rcode)[mism] == 1)
    assert firm.mean() > 0.99


def test_merge_without_adapter_is_the_dequantized_weight_and_requantizes_to_itself():
    h, o = 576, 192
    W, _, _, parts = _problem(h, o, 0, seed=11)
    print("merge r=0", flush=True)
    got = nf4.qlora_merge_adapter(W, None, None, 2.0, torch.float32)
    codes, absmax = nf4.qlora_merge_requantize(W, None, None, 2.0)
    torch.cuda.synchronize()
    wh = oracle.dequantized_weight(*parts[:4], h, o)
    assert np.array_equal(to_np(got).view(np.uint32), wh.view(np.uint32))
    pc, pa = oracle.quantize(wh.ravel())
    assert np.array_equal(to_np(codes), pc) and np.array_equal(to_np(codes), parts[0])
    assert np.array_equal(to_np(absmax).view(np.uint32), pa.view(np.uint32))


def test_merge_zero_scale_is_exact():
    h, o, r = 320, 256, 16
    W, L1, L2, parts = _problem(h, o, r, seed=21)
    print("merge s=0", flush=True)
    got = nf4.qlora_merge_adapter(W, L1, L2, 0.0, torch.float32)
    torch.cuda.synchronize()
    ref = oracle.merged_weight(*parts[:4], h, o, parts[4], parts[5], 0.0)
    assert np.array_equal(to_np(got).view(np.uint32), ref.view(np.uint32))


def test_merge_workload_shape():
    """A 7B MLP projection at full size (h = 4096, o = 11008, r = 64), compared in full."""
    h, o, r, s = 4096, 11008, 64, 2.0
    print("merge 4096x11008 r=64", flush=True)
    W, L1, L2, parts = _problem(h, o, r, seed=5)
    got = nf4.qlora_merge_adapter(W, L1, L2, s, torch.float32)
    torch.cuda.synchronize()
    ref = oracle.merged_weight(*parts[:4], h, o, parts[4], parts[5], s)
    err = np.abs(to_np(got).astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= _bound(parts, h, o, s))
