"""qlora_double_quant_noalloc (the allocation-free double quantization) against
qlora_double_quant with a caller workspace, through the C ABI: int8 scales,
second-level steps and the mean bit for bit, on two calls in a row (the second
smaller, so it runs after the first has left its partial sums in the shared
static array), then a third call interleaved with the workspace entry point."""
import ctypes

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_fine_nf4_amd as nf4  # noqa: E402

lib = nf4.lib
DEV = "cuda:0"


def scales(nb, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    a = (torch.randn(nb, device=DEV, generator=g).abs() * 0.02).float()
    a[:: max(1, nb // 7)] *= 10.0   # a few outliers
    return a


def run(nb, seed, noalloc):
    a = scales(nb, seed)
    qa = torch.empty(nb, dtype=torch.int8, device=DEV)
    s2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device=DEV)
    mean = torch.empty(1, dtype=torch.float32, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    if noalloc:
        rc = lib.qlora_double_quant_noalloc(p(a), nb, p(qa), p(s2), p(mean), st)
    else:
        ws = torch.empty(nf4.workspace_size(nf4.QLORA_OP_DOUBLE_QUANT, nb), dtype=torch.uint8, device=DEV)
        rc = lib.qlora_double_quant(p(a), nb, p(qa), p(s2), p(mean), p(ws), ws.numel(), st)
    assert rc == nf4.QLORA_OK, rc
    torch.cuda.synchronize()
    return a, qa.cpu().numpy(), s2.cpu().numpy().view(np.uint32), mean.cpu().numpy().view(np.uint32)


def same(x, y):
    return all(np.array_equal(u, v) for u, v in zip(x[1:], y[1:]))


@pytest.mark.parametrize("sizes", [(3_000_017, 1_000), (62_500_000, 257)])
def test_noalloc_double_quant_matches_workspace_entry_point(sizes):
    for i, nb in enumerate(sizes):
        print(f"noalloc double quant call {i} nb={nb}", flush=True)
        got = run(nb, 10 * i + nb % 97, noalloc=True)
        ref = run(nb, 10 * i + nb % 97, noalloc=False)
        assert same(got, ref), nb
        if nb <= 5000:  # small enough for the oracle too
            q, s2, mean = oracle.double_quant(got[0].cpu().numpy())
            assert np.array_equal(got[1], q) and np.array_equal(got[2], s2.view(np.uint32))
            assert got[3][0] == np.float32(mean).view(np.uint32)


def test_noalloc_interleaved_with_workspace_calls():
    print("noalloc double quant interleaved", flush=True)
    a = run(100_003, 5, noalloc=True)
    b = run(40_000, 6, noalloc=False)
    c = run(100_003, 5, noalloc=True)
    d = run(40_000, 6, noalloc=True)
    assert same(a, c) and same(b, d)
