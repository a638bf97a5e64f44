"""GPU parity of the codec entry points against the oracle: bit-exact packed
codes, float32 block scales, int8 scales, second-level steps, the mean, and
float32 / bf16 dequantized values."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_fine_nf4_amd as nf4  # noqa: E402

DEV = "cuda:0"
F32 = np.float32


def gpu_quantize(w: np.ndarray, bf16: bool = False):
    t = torch.from_numpy(w).to(DEV)
    if bf16:
        t = t.view(torch.bfloat16) if w.dtype == np.uint16 else t.to(torch.bfloat16)
    codes, absmax = nf4.qlora_quantize(t)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), absmax.cpu().numpy()


def check_quantize(w32: np.ndarray, label: str):
    p, a = gpu_quantize(w32)
    rp, ra = oracle.quantize(w32)
    assert np.array_equal(a.view(np.uint32), ra.view(np.uint32)), f"{label}: absmax differs"
    bad = np.flatnonzero(p != rp)
    assert bad.size == 0, f"{label}: {bad.size} code bytes differ, first at {bad[:5]}"


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 130, 511, 512, 513, 1000, 4097, 64 * 1000 + 37, 1 << 20])
def test_quantize_f32_sizes(n):
    print(f"quantize f32 n={n}", flush=True)
    w = (np.random.default_rng(n).standard_normal(n) * 0.02).astype(F32)
    check_quantize(w, f"n={n}")


@pytest.mark.parametrize("n", [1, 7, 64, 100, 4096 + 9, 1 << 20])
def test_quantize_bf16_sizes(n):
    print(f"quantize bf16 n={n}", flush=True)
    w = torch.from_numpy((np.random.default_rng(n + 1).standard_normal(n) * 0.02).astype(F32)).to(torch.bfloat16)
    bits = w.view(torch.int16).numpy().view(np.uint16)
    p, a = gpu_quantize(bits, bf16=True)
    rp, ra = oracle.quantize_bf16(bits)
    assert np.array_equal(a.view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(p, rp)


def test_quantize_special_blocks():
    print("quantize special blocks", flush=True)
    lv = oracle.nf4_levels()
    blocks = []
    blocks.append(np.zeros(64, F32))                                   # all zero
    b = np.zeros(64, F32); b[5] = -0.0; b[9] = 1e-45; blocks.append(b)  # denormal absmax
    b = np.full(64, -0.0, F32); b[0] = 0.3; blocks.append(b)            # negative zeros
    for a in (1.0, 0.02, 3.7e-30, 1e30, 2.0 ** -101, 2.0 ** 101, 1e-38):
        v = (lv * F32(a)).astype(F32)
        blocks.append(np.concatenate([v, v[::-1], v, v[::-1]]))        # every level x absmax
    mid = oracle.nf4_midpoints()
    b = np.zeros(64, F32); b[0] = 1.0; b[1:16] = mid.astype(F32); b[16:31] = -mid.astype(F32)  # ties at a = 1
    blocks.append(b)
    w = np.concatenate(blocks)
    check_quantize(w, "special")


def test_quantize_guard_bands():
    """Values packed around every decision boundary fp32(m_j * a) for many scales a:
    exercises the bucket table's guard bands and the exact fallback."""
    print("quantize guard bands", flush=True)
    rng = np.random.default_rng(42)
    mid = oracle.nf4_midpoints()
    blocks = []
    for a in np.concatenate([rng.uniform(0.001, 0.2, 400), 2.0 ** rng.uniform(-60, 60, 100)]).astype(F32):
        for j in range(15):
            c = np.float32(mid[j] * float(a))
            vals = [c]
            lo = hi = c
            for _ in range(31):
                lo = np.nextafter(lo, F32(-np.inf))
                hi = np.nextafter(hi, F32(np.inf))
                vals += [lo, hi]
            blk = np.array([a] + vals, F32)[:64]
            blocks.append(np.clip(blk, -a, a))
    w = np.concatenate(blocks)
    check_quantize(w, "guard bands")


def test_quantize_random_scales_large():
    print("quantize random scales", flush=True)
    rng = np.random.default_rng(3)
    nb = 1 << 15
    scales = (2.0 ** rng.uniform(-20, 10, nb)).astype(F32)
    w = (rng.standard_normal((nb, 64)) * scales[:, None]).astype(F32).ravel()
    w[rng.random(w.size) < 1e-3] = 0.0
    check_quantize(w, "random scales")


@pytest.mark.parametrize("nb", [1, 2, 255, 256, 257, 1000, 100003, 5000011])
def test_double_quant(nb):
    print(f"double quant nb={nb}", flush=True)
    rng = np.random.default_rng(nb)
    a = (np.abs(rng.standard_normal(nb)) * 0.03 + 0.005).astype(F32)
    if nb > 10:
        a[::97] = (2.0 ** rng.uniform(-140, 20, a[::97].size)).astype(F32)   # far-off exponents
        a[3] = 0.0
    q, s2, mean = nf4.qlora_double_quant(torch.from_numpy(a).to(DEV))
    torch.cuda.synchronize()
    rq, rs2, rmean = oracle.double_quant(a)
    assert mean.cpu().numpy()[0].view(np.uint32) == np.float32(rmean).view(np.uint32), (mean, rmean)
    assert np.array_equal(s2.cpu().numpy().view(np.uint32), rs2.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


def test_double_quant_exact_mean_extremes():
    print("double quant mean extremes", flush=True)
    one = F32(1.0)
    up = np.nextafter(one, F32(2))
    cases = [np.array([one, up], F32), np.array([1e30, 1e-30, 1e-30], F32),
             np.array([1e-45] * 5 + [3e-45], F32), np.full(70000, F32(0.0421)),
             np.array([3.4e38, 3.4e38, 1e-45], F32)]
    for a in cases:
        _, _, mean = nf4.qlora_double_quant(torch.from_numpy(a).to(DEV))
        torch.cuda.synchronize()
        assert mean.cpu().numpy()[0] == oracle.exact_mean_f32(a), a[:4]


@pytest.mark.parametrize("n", [1, 31, 32, 33, 64, 100, 4097, 64 * 777 + 13, 1 << 20])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize(n, out):
    print(f"dequantize n={n} {out}", flush=True)
    w = (np.random.default_rng(n + 7).standard_normal(n) * 0.02).astype(F32)
    p, a = oracle.quantize(w)
    q, s2, mean = oracle.double_quant(a)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    res = nf4.qlora_dequantize(t(p), t(q), t(s2), t(np.array([mean], F32)), n,
                               torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.dequantize(p, q, s2, mean, n, out=out)
    got = res.cpu()
    got = got.numpy() if out == "f32" else got.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got.view(np.uint32 if out == "f32" else np.uint16),
                          ref.view(np.uint32 if out == "f32" else np.uint16))


def test_codec_roundtrip_gpu_chain():
    """quantize -> double_quant -> dequantize entirely on the GPU vs the oracle chain."""
    print("codec chain", flush=True)
    w = wl.codec_chunk_f32(64 * 5000 + 40, seed=9)
    codes, absmax = nf4.qlora_quantize(torch.from_numpy(w).to(DEV))
    q, s2, mean = nf4.qlora_double_quant(absmax)
    d = nf4.qlora_dequantize(codes, q, s2, mean, w.size, torch.float32)
    torch.cuda.synchronize()
    p, a = oracle.quantize(w)
    rq, rs2, rmean = oracle.double_quant(a)
    ref = oracle.dequantize(p, rq, rs2, rmean, w.size)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_codec_full_size_sampled():
    """The bandwidth workload at full size (4e9 bf16 weights with heavy-tailed blocks):
    sampled blocks are checked bit-exactly against the oracle, the mean against the
    oracle's exact mean of all block scales, and sampled chunks of int8 scales."""
    n = wl.C4_CODEC_N
    print(f"codec full size n={n}", flush=True)
    w = wl.codec_weights_device(n, seed=0, device=DEV)
    codes, absmax = nf4.qlora_quantize(w)
    q, s2, mean = nf4.qlora_double_quant(absmax)
    out = nf4.qlora_dequantize(codes, q, s2, mean, n, torch.bfloat16)
    torch.cuda.synchronize()
    nb = n // 64
    rng = np.random.default_rng(1)
    blocks = np.unique(np.concatenate([rng.integers(0, nb, 3000), [0, nb - 1]]))
    idx = torch.from_numpy(blocks).to(DEV)
    wb = w.view(-1, 64)[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    cb = codes.view(-1, 32)[idx].cpu().numpy()
    ab = absmax[idx].cpu().numpy()
    for i in range(blocks.size):
        rp, ra = oracle.quantize_bf16(wb[i])
        assert ra[0].view(np.uint32) == ab[i].view(np.uint32)
        assert np.array_equal(rp, cb[i])
    a_all = absmax.cpu().numpy()
    assert mean.cpu().numpy()[0] == oracle.exact_mean_f32(a_all)
    mu = mean.cpu().numpy()[0]
    q_all = q.cpu().numpy()
    s2_all = s2.cpu().numpy()
    for ch in np.unique(np.concatenate([blocks // 256, [s2_all.size - 1]])):
        c = (a_all[ch * 256:(ch + 1) * 256] - mu).astype(F32)
        rq, rstep = oracle.int8_absmax_quantize(c)
        assert rstep.view(np.uint32) == s2_all[ch].view(np.uint32)
        assert np.array_equal(rq, q_all[ch * 256:(ch + 1) * 256])
    ob = out.view(-1, 64)[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    for i, b in enumerate(blocks):
        ref = oracle.dequantize(cb[i], q_all[b:b + 1], s2_all[b // 256:b // 256 + 1], mu, 64, out="bf16")
        assert np.array_equal(ref, ob[i])
