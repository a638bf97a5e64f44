"""Python binding of libqlora_nf4.so — the MI355X (gfx950) NF4 + LoRA linear layer.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory and the current stream.  The functions carry
the C ABI's names (include/qlora_nf4.h).  Importing this module loads the
library; if it has not been built, the import raises (there is no fallback).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch  # noqa: F401  (loads the HIP runtime the library then shares)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_nf4.so")

QLORA_OK, QLORA_ERR_INVALID_VALUE, QLORA_ERR_UNSUPPORTED, QLORA_ERR_LAUNCH, QLORA_ERR_INTERNAL = range(5)
QLORA_F32, QLORA_BF16 = 0, 1
QLORA_CB_NF4, QLORA_CB_INT4, QLORA_CB_FP4 = 0, 1, 2
CODEBOOKS = {"nf4": QLORA_CB_NF4, "int4": QLORA_CB_INT4, "fp4": QLORA_CB_FP4}
QLORA_OP_DOUBLE_QUANT, QLORA_OP_LINEAR_FWD, QLORA_OP_LINEAR_BWD = 0, 1, 2
BLOCK, CHUNK, MAX_RANK = 64, 256, 128

EXPORTED = ("qlora_quantize", "qlora_double_quant", "qlora_dequantize", "qlora_linear_fwd",
            "qlora_linear_bwd", "qlora_merge_adapter", "qlora_merge_requantize", "qlora_adamw_step",
            "qlora_quantize_cb", "qlora_dequantize_cb", "qlora_dequantize_nodq", "qlora_codebook_levels",
            "qlora_linear_fwd_cb", "qlora_linear_bwd_cb", "qlora_merge_adapter_cb", "qlora_merge_requantize_cb",
            "qlora_silu_gate_fwd", "qlora_silu_gate_bwd", "qlora_grad_sum", "qlora_double_quant_noalloc",
            "qlora_workspace_size", "qlora_stream_probe",
            "qlora_status_string", "qlora_nf4_levels", "qlora_set_timing_events")


class QloraError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib.qlora_status_string(status).decode()} (status {status})")
        self.status = status


class NF4WeightT(ctypes.Structure):
    """qlora_nf4_weight_t: four device pointers, then h and o."""
    _fields_ = [("codes", ctypes.c_void_p), ("qabsmax", ctypes.c_void_p), ("scale2", ctypes.c_void_p),
                ("mean", ctypes.c_void_p), ("h", ctypes.c_int64), ("o", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python bit_quantized_fine_nf4_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_int
    sz = ctypes.c_size_t
    L.qlora_quantize.argtypes = [vp, st, i64, vp, vp, vp]
    L.qlora_double_quant.argtypes = [vp, i64, vp, vp, vp, vp, sz, vp]
    L.qlora_double_quant_noalloc.argtypes = [vp, i64, vp, vp, vp, vp]
    L.qlora_dequantize.argtypes = [vp, vp, vp, vp, i64, vp, st, vp]
    L.qlora_quantize_cb.argtypes = [vp, st, i64, st, vp, vp, vp]
    L.qlora_dequantize_cb.argtypes = [vp, vp, vp, vp, i64, st, vp, st, vp]
    L.qlora_dequantize_nodq.argtypes = [vp, vp, i64, st, vp, st, vp]
    L.qlora_codebook_levels.argtypes = [st, ctypes.POINTER(ctypes.c_float)]
    L.qlora_linear_fwd.argtypes = [ctypes.POINTER(NF4WeightT), vp, i64, vp, vp, i32, f32, vp, vp, vp, sz, vp]
    L.qlora_linear_bwd.argtypes = [ctypes.POINTER(NF4WeightT), vp, vp, vp, i64, vp, vp, i32, f32, vp, vp, vp,
                                   vp, sz, vp]
    L.qlora_merge_adapter.argtypes = [ctypes.POINTER(NF4WeightT), vp, vp, i32, f32, vp, st, vp]
    L.qlora_merge_requantize.argtypes = [ctypes.POINTER(NF4WeightT), vp, vp, i32, f32, vp, vp, vp]
    W = ctypes.POINTER(NF4WeightT)
    L.qlora_linear_fwd_cb.argtypes = [W, st] + L.qlora_linear_fwd.argtypes[1:]
    L.qlora_linear_bwd_cb.argtypes = [W, st] + L.qlora_linear_bwd.argtypes[1:]
    L.qlora_merge_adapter_cb.argtypes = [W, st] + L.qlora_merge_adapter.argtypes[1:]
    L.qlora_merge_requantize_cb.argtypes = [W, st] + L.qlora_merge_requantize.argtypes[1:]
    L.qlora_silu_gate_fwd.argtypes = [vp, vp, i64, vp, vp]
    L.qlora_silu_gate_bwd.argtypes = [vp, vp, vp, i64, vp, vp, vp]
    L.qlora_grad_sum.argtypes = [ctypes.POINTER(vp), i32, i64, vp, vp]
    L.qlora_stream_probe.argtypes = [i32, i32, i32, i32, vp, vp, i64, vp]
    L.qlora_adamw_step.argtypes = [vp, vp, vp, vp, i64, i64, f32, f32, f32, f32, f32, vp, vp]
    L.qlora_workspace_size.argtypes = [st, i64, i64, i64, i32, ctypes.POINTER(sz)]
    L.qlora_status_string.argtypes = [st]
    L.qlora_status_string.restype = ctypes.c_char_p
    L.qlora_nf4_levels.argtypes = [ctypes.POINTER(ctypes.c_float)]
    L.qlora_set_timing_events.argtypes = [i32, vp, vp]
    for name in EXPORTED:
        if name != "qlora_status_string":
            getattr(L, name).restype = ctypes.c_int
    return L


lib = _load()


def _check(status: int, where: str):
    if status != QLORA_OK:
        raise QloraError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_check(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def nf4_levels() -> list:
    buf = (ctypes.c_float * 16)()
    _check(lib.qlora_nf4_levels(buf), "qlora_nf4_levels")
    return list(buf)


TIMED_GEMM_FWD, TIMED_GEMM_DX, TIMED_GEMV = 0, 1, 2


def _event_handle(ev):
    if ev is None:
        return None
    if hasattr(ev, "cuda_event"):          # torch.cuda.Event (recorded by the library, so read it
        return ctypes.c_void_p(ev.cuda_event)  # back with hipEventElapsedTime, not torch)
    return ctypes.c_void_p(ev.value if isinstance(ev, ctypes.c_void_p) else int(ev))


def qlora_set_timing_events(kernel: int, start=None, stop=None):
    """Record the hipEvent_t pair (start, stop) around later launches of `kernel`
    by this thread (None, None switches the hook off)."""
    _check(lib.qlora_set_timing_events(kernel, _event_handle(start), _event_handle(stop)),
           "qlora_set_timing_events")


def workspace_size(op: int, a: int, b: int = 0, c: int = 0, r: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.qlora_workspace_size(op, a, b, c, r, ctypes.byref(out)), "qlora_workspace_size")
    return out.value


@dataclasses.dataclass
class NF4Weight:
    """A frozen NF4 weight with double-quantized scales, logical shape h x o,
    stored in [o][h] order (PyTorch Linear.weight)."""
    codes: torch.Tensor    # uint8 [o*h/2]
    qabsmax: torch.Tensor  # int8 [o*h/64]
    scale2: torch.Tensor   # float32 [ceil(o*h/64/256)]
    mean: torch.Tensor     # float32 [1]
    h: int
    o: int
    codebook: int = QLORA_CB_NF4

    def as_ctypes(self) -> NF4WeightT:
        return NF4WeightT(self.codes.data_ptr(), self.qabsmax.data_ptr(), self.scale2.data_ptr(),
                          self.mean.data_ptr(), self.h, self.o)

    def call(self, name: str, *args):
        """Call entry point `name` on this weight: the NF4 entry point, or its `_cb` variant
        with the codebook for other codebooks."""
        wt = self.as_ctypes()
        if self.codebook == QLORA_CB_NF4:
            return getattr(lib, name)(ctypes.byref(wt), *args)
        return getattr(lib, name + "_cb")(ctypes.byref(wt), self.codebook, *args)


# ---------------------------------------------------------------------------
# The entry points
# ---------------------------------------------------------------------------

def codebook_levels(codebook: int = QLORA_CB_NF4) -> list:
    buf = (ctypes.c_float * 16)()
    _check(lib.qlora_codebook_levels(codebook, buf), "qlora_codebook_levels")
    return list(buf)


def qlora_quantize(w: torch.Tensor, codes: Optional[torch.Tensor] = None,
                   absmax: Optional[torch.Tensor] = None, codebook: int = QLORA_CB_NF4) -> Tuple[torch.Tensor, torch.Tensor]:
    """Blockwise 4-bit quantization (NF4 unless `codebook` says otherwise) of any float32/bf16
    GPU tensor (flattened)."""
    _dev_check(w)
    n = w.numel()
    dtype = {torch.float32: QLORA_F32, torch.bfloat16: QLORA_BF16}[w.dtype]
    if codes is None:
        codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=w.device)
    if absmax is None:
        absmax = torch.empty((n + BLOCK - 1) // BLOCK, dtype=torch.float32, device=w.device)
    if codebook == QLORA_CB_NF4:
        _check(lib.qlora_quantize(_ptr(w), dtype, n, _ptr(codes), _ptr(absmax), _stream(w.device)), "qlora_quantize")
    else:
        _check(lib.qlora_quantize_cb(_ptr(w), dtype, n, codebook, _ptr(codes), _ptr(absmax), _stream(w.device)),
               "qlora_quantize_cb")
    return codes, absmax


def qlora_double_quant(absmax: torch.Tensor, qabsmax: Optional[torch.Tensor] = None,
                       scale2: Optional[torch.Tensor] = None, mean: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None):
    """Double quantization of the float32 block scales -> (qabsmax int8, scale2 f32, mean f32[1])."""
    _dev_check(absmax)
    nb = absmax.numel()
    dev = absmax.device
    if qabsmax is None:
        qabsmax = torch.empty(nb, dtype=torch.int8, device=dev)
    if scale2 is None:
        scale2 = torch.empty((nb + CHUNK - 1) // CHUNK, dtype=torch.float32, device=dev)
    if mean is None:
        mean = torch.empty(1, dtype=torch.float32, device=dev)
    ws_bytes = workspace_size(QLORA_OP_DOUBLE_QUANT, nb)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(lib.qlora_double_quant(_ptr(absmax), nb, _ptr(qabsmax), _ptr(scale2), _ptr(mean), _ptr(workspace),
                                  workspace.numel(), _stream(dev)), "qlora_double_quant")
    return qabsmax, scale2, mean


def qlora_dequantize(codes: torch.Tensor, qabsmax: torch.Tensor, scale2: torch.Tensor, mean: torch.Tensor,
                     n: int, out_dtype: torch.dtype = torch.bfloat16,
                     out: Optional[torch.Tensor] = None, codebook: int = QLORA_CB_NF4) -> torch.Tensor:
    """Rebuild n weights as float32 or bf16."""
    _dev_check(codes, qabsmax, scale2, mean)
    dt = {torch.float32: QLORA_F32, torch.bfloat16: QLORA_BF16}[out_dtype]
    if out is None:
        out = torch.empty(n, dtype=out_dtype, device=codes.device)
    if codebook == QLORA_CB_NF4:
        _check(lib.qlora_dequantize(_ptr(codes), _ptr(qabsmax), _ptr(scale2), _ptr(mean), n, _ptr(out), dt,
                                    _stream(codes.device)), "qlora_dequantize")
    else:
        _check(lib.qlora_dequantize_cb(_ptr(codes), _ptr(qabsmax), _ptr(scale2), _ptr(mean), n, codebook,
                                       _ptr(out), dt, _stream(codes.device)), "qlora_dequantize_cb")
    return out


def qlora_dequantize_nodq(codes: torch.Tensor, absmax: torch.Tensor, n: int, out_dtype: torch.dtype = torch.bfloat16,
                          out: Optional[torch.Tensor] = None, codebook: int = QLORA_CB_NF4) -> torch.Tensor:
    """Rebuild n weights from the float32 block scales (no double quantization)."""
    _dev_check(codes, absmax)
    dt = {torch.float32: QLORA_F32, torch.bfloat16: QLORA_BF16}[out_dtype]
    if out is None:
        out = torch.empty(n, dtype=out_dtype, device=codes.device)
    _check(lib.qlora_dequantize_nodq(_ptr(codes), _ptr(absmax), n, codebook, _ptr(out), dt, _stream(codes.device)),
           "qlora_dequantize_nodq")
    return out


def quantize_weight(w_oh: torch.Tensor, codebook: int = QLORA_CB_NF4) -> NF4Weight:
    """quantize + double_quant of a [o][h] float32/bf16 weight."""
    o, h = w_oh.shape
    codes, absmax = qlora_quantize(w_oh, codebook=codebook)
    qa, s2, mean = qlora_double_quant(absmax)
    return NF4Weight(codes, qa, s2, mean, h, o, codebook)


def qlora_linear_fwd(W: NF4Weight, X: torch.Tensor, L1: Optional[torch.Tensor], L2: Optional[torch.Tensor],
                     s: float, Y: Optional[torch.Tensor] = None, T: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """Y = X·W_hat + s·(X·L1)·L2 -> (Y bf16 [M][o], T bf16 [M][r] or None)."""
    _dev_check(X, L1, L2)
    M = X.shape[0]
    r = 0 if L1 is None else L1.shape[1]
    dev = X.device
    if Y is None:
        Y = torch.empty(M, W.o, dtype=torch.bfloat16, device=dev)
    if T is None and r:
        T = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
    ws_bytes = workspace_size(QLORA_OP_LINEAR_FWD, M, W.h, W.o, r)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(W.call("qlora_linear_fwd", _ptr(X), M, _ptr(L1), _ptr(L2), r, float(s), _ptr(Y), _ptr(T),
                  _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(dev)),
           "qlora_linear_fwd")
    return Y, T


def qlora_merge_adapter(W: NF4Weight, L1: Optional[torch.Tensor], L2: Optional[torch.Tensor], s: float,
                        out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense merged weight W' = W_hat + s·L1·L2 in [o][h] storage (float32 or bf16)."""
    _dev_check(L1, L2)
    r = 0 if L1 is None else L1.shape[1]
    dt = {torch.float32: QLORA_F32, torch.bfloat16: QLORA_BF16}[out_dtype]
    if out is None:
        out = torch.empty(W.o, W.h, dtype=out_dtype, device=W.codes.device)
    _check(W.call("qlora_merge_adapter", _ptr(L1), _ptr(L2), r, float(s), _ptr(out), dt, _stream(W.codes.device)),
           "qlora_merge_adapter")
    return out


def qlora_merge_requantize(W: NF4Weight, L1: Optional[torch.Tensor], L2: Optional[torch.Tensor], s: float,
                           codes: Optional[torch.Tensor] = None, absmax: Optional[torch.Tensor] = None):
    """NF4 codes and float32 block absmax of the merged weight -> (codes, absmax)."""
    _dev_check(L1, L2)
    r = 0 if L1 is None else L1.shape[1]
    dev = W.codes.device
    n = W.h * W.o
    if codes is None:
        codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    if absmax is None:
        absmax = torch.empty(n // BLOCK, dtype=torch.float32, device=dev)
    _check(W.call("qlora_merge_requantize", _ptr(L1), _ptr(L2), r, float(s), _ptr(codes), _ptr(absmax),
                  _stream(dev)), "qlora_merge_requantize")
    return codes, absmax


def qlora_adamw_step(param: torch.Tensor, grad: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                     step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                     weight_decay: float = 0.0, param_bf16: Optional[torch.Tensor] = None,
                     device=None) -> None:
    """AdamW step on float32 `param` (in place, with its moments).  Each tensor is a
    contiguous float32 GPU tensor or a pinned host tensor (optimizer state kept in CPU RAM);
    `device` names the GPU whose current stream runs the step (default: param's, else cuda:0)."""
    ts = (param, grad, exp_avg, exp_avg_sq)
    for t in ts + (param_bf16,):
        if t is None:
            continue
        if not t.is_contiguous() or not (t.is_cuda or t.is_pinned()):
            raise ValueError("tensors must be contiguous, on the GPU or in pinned host memory")
    if any(t.dtype != torch.float32 for t in ts) or (param_bf16 is not None and param_bf16.dtype != torch.bfloat16):
        raise ValueError("param, grad and moments are float32; param_bf16 is bf16")
    n = param.numel()
    if any(t.numel() != n for t in ts[1:]) or (param_bf16 is not None and param_bf16.numel() != n):
        raise ValueError("all arrays must have param's size")
    if device is None:
        device = param.device if param.is_cuda else torch.device("cuda:0")
    _check(lib.qlora_adamw_step(_ptr(param), _ptr(grad), _ptr(exp_avg), _ptr(exp_avg_sq), n, int(step), float(lr),
                                float(beta1), float(beta2), float(eps), float(weight_decay), _ptr(param_bf16),
                                _stream(device)), "qlora_adamw_step")


def qlora_linear_bwd(W: NF4Weight, X: Optional[torch.Tensor], T: Optional[torch.Tensor], dY: torch.Tensor,
                     L1: Optional[torch.Tensor], L2: Optional[torch.Tensor], s: float,
                     dX: Optional[torch.Tensor] = None, dL1: Optional[torch.Tensor] = None,
                     dL2: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Backward through the frozen NF4 weight -> (dX bf16 [M][h], dL1 f32 [h][r], dL2 f32 [r][o])."""
    _dev_check(X, T, dY, L1, L2)
    M = dY.shape[0]
    r = 0 if L1 is None else L1.shape[1]
    dev = dY.device
    if dX is None:
        dX = torch.empty(M, W.h, dtype=torch.bfloat16, device=dev)
    if r and dL1 is None:
        dL1 = torch.empty(W.h, r, dtype=torch.float32, device=dev)
    if r and dL2 is None:
        dL2 = torch.empty(r, W.o, dtype=torch.float32, device=dev)
    ws_bytes = workspace_size(QLORA_OP_LINEAR_BWD, M, W.h, W.o, r)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(W.call("qlora_linear_bwd", _ptr(X), _ptr(T), _ptr(dY), M, _ptr(L1), _ptr(L2), r, float(s),
                  _ptr(dX), _ptr(dL1), _ptr(dL2), _ptr(workspace),
                  0 if workspace is None else workspace.numel(), _stream(dev)),
           "qlora_linear_bwd")
    return dX, dL1, dL2


# ---------------------------------------------------------------------------
# Block glue between the linears
# ---------------------------------------------------------------------------

def _same(*ts):
    n = ts[0].numel()
    for t in ts:
        if t.dtype != torch.bfloat16 or t.numel() != n:
            raise ValueError("glue tensors are bf16 of one size")
    return n


def qlora_silu_gate_fwd(G: torch.Tensor, U: torch.Tensor, H: Optional[torch.Tensor] = None) -> torch.Tensor:
    """H = SiLU(G) * U (bf16, elementwise)."""
    _dev_check(G, U, H)
    if H is None:
        H = torch.empty_like(G)
    n = _same(G, U, H)
    _check(lib.qlora_silu_gate_fwd(_ptr(G), _ptr(U), n, _ptr(H), _stream(G.device)), "qlora_silu_gate_fwd")
    return H


def qlora_silu_gate_bwd(G: torch.Tensor, U: torch.Tensor, dH: torch.Tensor, dG: Optional[torch.Tensor] = None,
                        dU: Optional[torch.Tensor] = None):
    """(dG, dU) of H = SiLU(G) * U for the upstream gradient dH."""
    _dev_check(G, U, dH, dG, dU)
    dG = torch.empty_like(G) if dG is None else dG
    dU = torch.empty_like(U) if dU is None else dU
    n = _same(G, U, dH, dG, dU)
    _check(lib.qlora_silu_gate_bwd(_ptr(G), _ptr(U), _ptr(dH), n, _ptr(dG), _ptr(dU), _stream(G.device)),
           "qlora_silu_gate_bwd")
    return dG, dU


def qlora_stream_probe(rd: int, wr: int, src: torch.Tensor, dst: torch.Tensor, n_tiles: int,
                       depth: int = 2, blocks: int = 0) -> None:
    """Measurement helper: stream n_tiles tiles of rd KB read and wr KB written, depth tiles per
    wave and pass, `blocks` workgroups (0: the library's default) (see the C header)."""
    _dev_check(src, dst)
    if src.numel() * src.element_size() < n_tiles * 1024 * rd or dst.numel() * dst.element_size() < max(16, n_tiles * 1024 * wr):
        raise ValueError("qlora_stream_probe: buffers too small for n_tiles")
    _check(lib.qlora_stream_probe(rd, wr, depth, blocks, _ptr(src), _ptr(dst), n_tiles, _stream(src.device)),
           "qlora_stream_probe")


def qlora_grad_sum(parts, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = parts[0] + ... + parts[k-1] (bf16, float32 sum in order, one rounding)."""
    parts = list(parts)
    _dev_check(*parts, out)
    if out is None:
        out = torch.empty_like(parts[0])
    n = _same(*parts, out)
    arr = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    _check(lib.qlora_grad_sum(arr, len(parts), n, _ptr(out), _stream(out.device)), "qlora_grad_sum")
    return out
