"""Helpers shared by the GPU parity tests: error metrics and oracle pipelines."""
from __future__ import annotations

import numpy as np
import torch

import oracle

REL_FROB_TOL = 1e-2      # relative Frobenius error bound for bf16 outputs vs the float64 oracle
MAX_ABS_TOL = 2e-2       # max-abs error bound, as a fraction of max|reference|


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / (den if den > 0 else 1.0)
    mx = np.abs(ref).max() if ref.size else 0.0
    mabs = np.abs(got - ref).max() / (mx if mx > 0 else 1.0) if ref.size else 0.0
    return float(rel), float(mabs)


def assert_close(name, got, ref):
    rel, mabs = errors(got, ref)
    print(f"  {name}: rel_frob={rel:.3e} max_abs/max|ref|={mabs:.3e}", flush=True)
    assert rel <= REL_FROB_TOL and mabs <= MAX_ABS_TOL, (name, rel, mabs)
    return rel, mabs


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def oracle_weight(w_oh: torch.Tensor) -> np.ndarray:
    """The oracle's own float32 reconstruction of a [o][h] weight (quantize, DQ, dequant)."""
    w = w_oh.detach().cpu()
    if w.dtype == torch.bfloat16:
        w = w.float()
    o, h = w.shape
    p, a = oracle.quantize(w.numpy().ravel())
    q, s2, mean = oracle.double_quant(a)
    return oracle.dequantized_weight(p, q, s2, mean, h, o)
