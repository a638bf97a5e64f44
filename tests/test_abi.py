"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, builds the same NF4 codebook as the oracle (independently),
sizes workspaces, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora_nf4.h")

nf4 = pytest.importorskip("bit_quantized_fine_nf4_amd")
lib = nf4.lib

FAKE = ctypes.c_void_p(0x100000)        # 16-byte aligned, never dereferenced (calls fail validation first)
ODD = ctypes.c_void_p(0x100002)         # misaligned


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qlora_\w+)\s*\(", text, re.M)))


def test_header_functions_are_exported():
    declared = header_functions()
    assert {"qlora_quantize", "qlora_double_quant", "qlora_dequantize", "qlora_linear_fwd",
            "qlora_linear_bwd"} <= set(declared)
    out = subprocess.run(["nm", "-D", "--defined-only", nf4.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (qlora_\w+)", out))
    assert set(declared) <= exported
    for name in declared:
        assert hasattr(lib, name)
    assert set(nf4.EXPORTED) == set(declared)


def test_library_codebook_matches_oracle_bitwise():
    lv = np.array(nf4.nf4_levels(), dtype=np.float32)
    assert np.array_equal(lv.view(np.uint32), oracle.nf4_levels().view(np.uint32))


def test_status_strings():
    for s in range(5):
        assert lib.qlora_status_string(s)
    assert b"invalid" in lib.qlora_status_string(1)


def test_workspace_sizes():
    assert nf4.workspace_size(nf4.QLORA_OP_DOUBLE_QUANT, 1000) % 256 == 0
    assert nf4.workspace_size(nf4.QLORA_OP_LINEAR_FWD, 16, 1024, 1024, 0) == 0
    # the few-token backward keeps float32 partial sums of dX even without an adapter
    assert nf4.workspace_size(nf4.QLORA_OP_LINEAR_BWD, 16, 1024, 1024, 0) >= 16 * 1024 * 4
    assert nf4.workspace_size(nf4.QLORA_OP_LINEAR_BWD, 17, 1024, 1024, 0) == 0
    for op in (nf4.QLORA_OP_LINEAR_FWD, nf4.QLORA_OP_LINEAR_BWD):
        b = nf4.workspace_size(op, 2048, 4096, 4096, 16)
        assert b > 0 and b % 256 == 0
    with pytest.raises(nf4.QloraError):
        nf4.workspace_size(nf4.QLORA_OP_LINEAR_FWD, 0, 64, 64, 8)
    with pytest.raises(nf4.QloraError):
        nf4.workspace_size(nf4.QLORA_OP_LINEAR_FWD, 8, 64, 64, 129)
    assert lib.qlora_workspace_size(7, 1, 1, 1, 0, ctypes.byref(ctypes.c_size_t())) == nf4.QLORA_ERR_INVALID_VALUE


INV = nf4.QLORA_ERR_INVALID_VALUE


def test_quantize_rejects_bad_arguments():
    q = lib.qlora_quantize
    assert q(None, 0, 10, FAKE, FAKE, None) == INV
    assert q(FAKE, 0, 0, FAKE, FAKE, None) == INV
    assert q(FAKE, 0, -5, FAKE, FAKE, None) == INV
    assert q(FAKE, 2, 10, FAKE, FAKE, None) == INV
    assert q(ODD, 0, 10, FAKE, FAKE, None) == INV
    assert q(FAKE, 1, 10, None, FAKE, None) == INV
    assert q(FAKE, 1, 10, FAKE, None, None) == INV


def test_double_quant_and_dequant_reject_bad_arguments():
    dq = lib.qlora_double_quant
    assert dq(FAKE, 0, FAKE, FAKE, FAKE, FAKE, 4096, None) == INV
    assert dq(FAKE, 1 << 32, FAKE, FAKE, FAKE, FAKE, 4096, None) == INV
    assert dq(FAKE, 100, FAKE, FAKE, FAKE, FAKE, 8, None) == INV          # workspace too small
    assert dq(FAKE, 100, FAKE, FAKE, FAKE, None, 4096, None) == INV
    assert dq(ODD, 100, FAKE, FAKE, FAKE, FAKE, 4096, None) == INV
    de = lib.qlora_dequantize
    assert de(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, None) == INV
    assert de(FAKE, FAKE, FAKE, FAKE, 10, FAKE, 5, None) == INV
    assert de(FAKE, FAKE, FAKE, None, 10, FAKE, 0, None) == INV
    assert de(FAKE, FAKE, FAKE, FAKE, 10, ODD, 1, None) == INV


def weight(h=128, o=64, codes=FAKE):
    return nf4.NF4WeightT(codes.value if codes is not None else None, FAKE.value, FAKE.value, FAKE.value, h, o)


def test_linear_rejects_bad_arguments():
    fwd, bwd = lib.qlora_linear_fwd, lib.qlora_linear_bwd
    ok = weight()
    ws = 1 << 30
    args = lambda W, X=FAKE, M=4, L1=FAKE, L2=FAKE, r=8, Y=FAKE, T=FAKE, w=FAKE: \
        fwd(ctypes.byref(W), X, M, L1, L2, r, 2.0, Y, T, w, ws, None)
    assert args(weight(h=100)) == INV                   # h not a multiple of 64
    assert args(weight(o=0)) == INV
    assert args(weight(codes=None)) == INV
    assert args(weight(codes=ODD)) == INV
    assert args(ok, M=0) == INV
    assert args(ok, r=-1) == INV
    assert args(ok, r=129) == INV
    assert args(ok, L1=None) == INV
    assert args(ok, T=None) == INV
    assert args(ok, X=None) == INV
    assert args(ok, X=ODD) == INV
    assert args(ok, w=None) == INV                      # r > 0 needs a workspace
    assert fwd(ctypes.byref(ok), FAKE, 4, FAKE, FAKE, 8, 2.0, FAKE, FAKE, FAKE, 16, None) == INV
    b = lambda W=ok, X=FAKE, T=FAKE, dY=FAKE, M=4, r=8, dX=FAKE, dL1=FAKE: \
        bwd(ctypes.byref(W), X, T, dY, M, FAKE, FAKE, r, 2.0, dX, dL1, FAKE, FAKE, ws, None)
    assert b(dY=None) == INV
    assert b(dX=None) == INV
    assert b(X=None) == INV
    assert b(T=None) == INV
    assert b(dL1=None) == INV
    assert b(M=-1) == INV
    assert b(W=weight(h=64, o=65)) == INV


def test_merge_rejects_bad_arguments():
    mg, rq = lib.qlora_merge_adapter, lib.qlora_merge_requantize
    ok = weight()
    m = lambda W=ok, L1=FAKE, L2=FAKE, r=8, out=FAKE, dt=0: mg(ctypes.byref(W), L1, L2, r, 2.0, out, dt, None)
    assert m(weight(h=100)) == INV
    assert m(weight(codes=ODD)) == INV
    assert m(out=None) == INV
    assert m(out=ODD) == INV
    assert m(dt=2) == INV
    assert m(r=-1) == INV
    assert m(r=129) == INV
    assert m(L1=None) == INV
    assert m(L2=ODD) == INV
    q = lambda W=ok, L1=FAKE, L2=FAKE, r=8, c=FAKE, a=FAKE: rq(ctypes.byref(W), L1, L2, r, 2.0, c, a, None)
    assert q(c=None) == INV
    assert q(a=None) == INV
    assert q(c=ODD) == INV
    assert q(L2=None) == INV
    assert q(r=200) == INV
    assert q(weight(o=32)) == INV


def test_adamw_rejects_bad_arguments():
    ad = lib.qlora_adamw_step
    a = lambda p=FAKE, g=FAKE, m=FAKE, v=FAKE, n=10, t=1, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0, bf=None: \
        ad(p, g, m, v, n, t, lr, b1, b2, eps, wd, bf, None)
    assert a(n=0) == INV
    assert a(t=0) == INV
    assert a(p=None) == INV
    assert a(v=None) == INV
    assert a(g=ODD) == INV
    assert a(bf=ODD) == INV
    assert a(b1=1.0) == INV
    assert a(b2=-0.1) == INV
    assert a(eps=0.0) == INV
    assert a(lr=-1.0) == INV
    assert a(wd=float("nan")) == INV


@pytest.mark.parametrize("name", ["nf4", "int4", "fp4"])
def test_codebook_levels_match_oracle_bitwise(name):
    got = np.array(nf4.codebook_levels(nf4.CODEBOOKS[name]), np.float32)
    assert np.array_equal(got.view(np.uint32), oracle.codebooks.levels(name).view(np.uint32))


def test_codebook_entry_points_reject_bad_arguments():
    buf = (ctypes.c_float * 16)()
    assert lib.qlora_codebook_levels(3, buf) == INV
    assert lib.qlora_codebook_levels(-1, buf) == INV
    assert lib.qlora_quantize_cb(FAKE, 0, 10, 3, FAKE, FAKE, None) == INV
    assert lib.qlora_quantize_cb(FAKE, 0, 0, 1, FAKE, FAKE, None) == INV
    assert lib.qlora_dequantize_cb(FAKE, FAKE, FAKE, FAKE, 10, 7, FAKE, 0, None) == INV
    assert lib.qlora_dequantize_nodq(FAKE, None, 10, 1, FAKE, 0, None) == INV
    assert lib.qlora_dequantize_nodq(FAKE, FAKE, 10, 1, ODD, 0, None) == INV
    assert lib.qlora_dequantize_nodq(FAKE, FAKE, 0, 1, FAKE, 0, None) == INV
    W = weight()
    for cb in (3, -1):
        assert lib.qlora_merge_adapter_cb(ctypes.byref(W), cb, FAKE, FAKE, 8, 1.0, FAKE, 0, None) == INV
        assert lib.qlora_merge_requantize_cb(ctypes.byref(W), cb, FAKE, FAKE, 8, 1.0, FAKE, FAKE, None) == INV
        assert lib.qlora_linear_fwd_cb(ctypes.byref(W), cb, FAKE, 4, FAKE, FAKE, 8, 2.0, FAKE, FAKE, FAKE,
                                       1 << 30, None) == INV
        assert lib.qlora_linear_bwd_cb(ctypes.byref(W), cb, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 8, 2.0, FAKE, FAKE,
                                       FAKE, FAKE, 1 << 30, None) == INV


LAYOUT_PROBE = r"""
#include <stddef.h>
#include <stdio.h>
#include "qlora_nf4.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu\n", sizeof(qlora_nf4_weight_t), offsetof(qlora_nf4_weight_t, codes),
         offsetof(qlora_nf4_weight_t, qabsmax), offsetof(qlora_nf4_weight_t, scale2),
         offsetof(qlora_nf4_weight_t, mean), offsetof(qlora_nf4_weight_t, h), offsetof(qlora_nf4_weight_t, o));
  return 0;
}
"""


def test_weight_struct_layout(tmp_path):
    """The weight descriptor is the boundary's plain struct: four pointers (codes,
    qabsmax, scale2, mean) then the int64 sizes h and o, 48 bytes.  Checked as a C
    compiler sees the header, and against the binding's ctypes mirror."""
    src = tmp_path / "layout.c"
    src.write_text(LAYOUT_PROBE)
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got == [48, 0, 8, 16, 24, 32, 40]
    assert ctypes.sizeof(nf4.NF4WeightT) == 48
    assert [getattr(nf4.NF4WeightT, f).offset for f in ("codes", "qabsmax", "scale2", "mean", "h", "o")] == \
        [0, 8, 16, 24, 32, 40]


def test_linear_bwd_token_split_bound():
    """The adapter-gradient reduction splits the tokens into chunks whose operand slab
    (chunk rows of max(h, o) bf16 values) stays below 2^31 bytes.  Observable on the host:
    the workspace holds one float32 partial tile per split, so its size grows with the
    number of splits once M passes the cap; a shape needing more than 65535 splits is
    rejected before anything is launched.  (r = 100 here: ranks up to 16 take the
    one-pass kernel while every token's slab fits 32-bit offsets; checked below.)"""
    h, o, r = 22016, 8192, 100
    rp16, rp64 = 112, 128
    cap = (0x7FFFFFF0 // (2 * h)) // 64 * 64          # 48768 tokens per split
    ws = lambda M, r=r: nf4.workspace_size(nf4.QLORA_OP_LINEAR_BWD, M, h, o, r)
    part = (h + o) * rp16 * 4      # one split's float32 partial tiles
    per_token = (rp16 + rp64) * 2  # U and s*U, bf16, r padded to 16 and to 64
    for M in (cap, 5 * cap + 1, 40 * cap, 100 * cap):
        # without the cap about 2 splits would do (256 workgroups over 236 tiles)
        splits = -(-M // cap)
        assert ws(M) >= M * per_token + splits * part, M
    assert ws(cap) < cap * per_token + 4 * part
    # r = 16: no partial tiles while M rows of the wider operand stay below 2^31 bytes
    # (one pass over every token), split partials past that
    one = (0x7FFF0000 - 1) // (2 * h)
    fixed = h * 64 * 2                                # L1 padded to 64 columns
    assert ws(one, 16) < one * (16 + 64) * 2 + fixed + 4096
    assert ws(one + 1, 16) >= (one + 1) * (16 + 64) * 2 + (h + o) * 16 * 4
    big = weight(h=1 << 20, o=64)
    M = 1 << 31                                         # 1024-token chunks -> 2^21 splits: unsupported
    st = lib.qlora_linear_bwd(ctypes.byref(big), FAKE, FAKE, FAKE, M, FAKE, FAKE, 8, 1.0, FAKE, FAKE, FAKE, FAKE,
                              ctypes.c_size_t(1 << 62), None)
    assert st == nf4.QLORA_ERR_UNSUPPORTED


def test_glue_entry_points_reject_bad_arguments():
    f, b, sm = lib.qlora_silu_gate_fwd, lib.qlora_silu_gate_bwd, lib.qlora_grad_sum
    assert f(None, FAKE, 10, FAKE, None) == INV
    assert f(FAKE, FAKE, 0, FAKE, None) == INV
    assert f(FAKE, ODD, 10, FAKE, None) == INV
    assert b(FAKE, FAKE, FAKE, 10, FAKE, None, None) == INV
    assert b(FAKE, FAKE, FAKE, 10, FAKE, FAKE, None) == INV        # dG and dU the same buffer
    assert b(FAKE, FAKE, ODD, 10, FAKE, ctypes.c_void_p(0x200000), None) == INV
    arr = (ctypes.c_void_p * 9)(*([FAKE.value] * 9))
    assert sm(arr, 0, 10, FAKE, None) == INV
    assert sm(arr, 9, 10, FAKE, None) == INV
    assert sm(arr, 2, 0, FAKE, None) == INV
    assert sm(None, 2, 10, FAKE, None) == INV
    bad = (ctypes.c_void_p * 2)(FAKE.value, ODD.value)
    assert sm(bad, 2, 10, FAKE, None) == INV


def test_double_quant_noalloc_rejects_bad_arguments():
    dq = lib.qlora_double_quant_noalloc
    assert dq(None, 10, FAKE, FAKE, FAKE, None) == INV
    assert dq(FAKE, 0, FAKE, FAKE, FAKE, None) == INV
    assert dq(FAKE, 1 << 32, FAKE, FAKE, FAKE, None) == INV
    assert dq(ODD, 10, FAKE, FAKE, FAKE, None) == INV
    assert dq(FAKE, 10, FAKE, None, FAKE, None) == INV


def test_stream_probe_rejects_bad_arguments():
    sp = lib.qlora_stream_probe
    assert sp(2, 1, 2, 0, FAKE, FAKE, 4, None) == INV       # only (1, 0), (4, 1), (1, 4)
    assert sp(1, 1, 2, 0, FAKE, FAKE, 4, None) == INV
    assert sp(1, 0, 3, 0, FAKE, FAKE, 4, None) == INV       # depth 1, 2, 4 or 8
    assert sp(1, 0, 16, 0, FAKE, FAKE, 4, None) == INV
    assert sp(1, 0, 2, -1, FAKE, FAKE, 4, None) == INV      # blocks in [0, 2^20]
    assert sp(1, 0, 2, (1 << 20) + 1, FAKE, FAKE, 4, None) == INV
    assert sp(1, 0, 2, 0, None, FAKE, 4, None) == INV
    assert sp(4, 1, 2, 0, FAKE, None, 4, None) == INV
    assert sp(1, 4, 2, 0, ODD, FAKE, 4, None) == INV
    assert sp(1, 4, 2, 0, FAKE, ODD, 4, None) == INV
    assert sp(1, 0, 2, 0, FAKE, FAKE, 0, None) == INV
    assert sp(1, 0, 2, 0, FAKE, FAKE, 1 << 40, None) == INV