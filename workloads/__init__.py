"""Seeded synthetic inputs for the NF4 + LoRA linear layer.

This module only draws random numbers and shapes them; it holds none of the
quantization or matmul arithmetic.  Both the CPU oracle (through the tests and
the bench) and the HIP path consume exactly the tensors produced here.

Workloads follow the shapes of the QLoRA pages: a frozen base weight W of shape
h x o (stored as PyTorch's [o][h] ``Linear.weight`` order), LoRA factors L1 (h x r)
and L2 (r x o), a scalar s, bf16 activations.  Pretrained weights are stood in
for by zero-mean normal draws ("bell-curved", "concentrated near zero"), and
outliers by sparse x10 entries or heavy-tailed Student-t blocks.

Every draw is seeded by ``(workload id, tensor id, linear index, chunk)``:
tensor ids are 0 = W, 1 = outlier mask, 2 = L1, 3 = L2, 4 = X, 5 = dY,
6 = stand-ins.  Values are drawn in float64, rounded to float32, and (for bf16
tensors) rounded once more by PyTorch's round-to-nearest-even cast.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

TENSOR_W, TENSOR_MASK, TENSOR_L1, TENSOR_L2, TENSOR_X, TENSOR_DY, TENSOR_AUX = range(7)


@dataclasses.dataclass(frozen=True)
class LinearShape:
    """One NF4 linear: input width h, output width o, LoRA rank r, scale s."""
    name: str
    h: int
    o: int
    r: int
    s: float


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    linears: tuple
    tokens: int
    w_std: float = 0.02
    outlier_p: float = 0.0      # per-entry probability of a x10 outlier
    lora_std: float = 0.01


# The five workloads.  Shapes are LLaMA-7B / LLaMA-65B projection sizes.
C1 = Workload(0, "linear_h1024_o1024_m16_r8",
              (LinearShape("lin", 1024, 1024, 8, 2.0),), tokens=16)
C2 = Workload(1, "attn_proj_h4096_o4096_m2048_r16",
              (LinearShape("proj", 4096, 4096, 16, 2.0),), tokens=2048, outlier_p=0.001)
C3 = Workload(2, "llama7b_mlp_h4096_f11008_m4096_r64",
              (LinearShape("gate", 4096, 11008, 64, 0.25),
               LinearShape("up", 4096, 11008, 64, 0.25),
               LinearShape("down", 11008, 4096, 64, 0.25)), tokens=4096)
C4_GEMV = Workload(3, "gemv_h8192_o28672",
                   (LinearShape("gemv", 8192, 28672, 0, 1.0),), tokens=16)
C5 = Workload(4, "llama65b_block_d8192_f22016_m2048_r64",
              (LinearShape("q", 8192, 8192, 64, 0.25),
               LinearShape("k", 8192, 8192, 64, 0.25),
               LinearShape("v", 8192, 8192, 64, 0.25),
               LinearShape("o", 8192, 8192, 64, 0.25),
               LinearShape("gate", 8192, 22016, 64, 0.25),
               LinearShape("up", 8192, 22016, 64, 0.25),
               LinearShape("down", 22016, 8192, 64, 0.25)), tokens=2048)
C4_CODEC_N = 4_000_000_000        # weights in the bandwidth-bound codec workload
C4_CODEC_WID = 3
C4_T_BLOCK_P = 0.01               # probability that a 64-block is heavy tailed
C4_GEMV_TOKENS = (1, 4, 16)

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4_GEMV, C5)}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def normal_f32(shape, std: float, *key: int) -> np.ndarray:
    """float32 array of N(0, std^2) draws (std is the standard deviation)."""
    x = _rng(*key).standard_normal(size=shape)
    return (x * std).astype(np.float32)


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 numpy -> bf16 CPU tensor (PyTorch's RNE cast)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def base_weight(wl: Workload, li: int) -> torch.Tensor:
    """Frozen base weight in [o][h] order, float32 CPU tensor.

    Entries are N(0, w_std^2); with probability ``outlier_p`` an entry is
    multiplied by 10 (sparse outliers).
    """
    ls = wl.linears[li]
    w = normal_f32((ls.o, ls.h), wl.w_std, wl.wid, TENSOR_W, li, 0)
    if wl.outlier_p > 0:
        mask = _rng(wl.wid, TENSOR_MASK, li, 0).random(size=w.shape) < wl.outlier_p
        w = np.where(mask, w * np.float32(10.0), w).astype(np.float32)
    return torch.from_numpy(w)


def lora_factors(wl: Workload, li: int):
    """(L1 [h][r], L2 [r][o]) bf16 CPU tensors, N(0, lora_std^2)."""
    ls = wl.linears[li]
    if ls.r == 0:
        return None, None
    l1 = normal_f32((ls.h, ls.r), wl.lora_std, wl.wid, TENSOR_L1, li, 0)
    l2 = normal_f32((ls.r, ls.o), wl.lora_std, wl.wid, TENSOR_L2, li, 0)
    return to_bf16(l1), to_bf16(l2)


def activations(wl: Workload, li: int, tokens: Optional[int] = None, width: Optional[int] = None,
                tensor: int = TENSOR_X) -> torch.Tensor:
    """bf16 CPU tensor [tokens][width] of N(0, 1) draws (X, dY or stand-ins)."""
    m = wl.tokens if tokens is None else tokens
    if width is None:
        width = wl.linears[li].h if tensor == TENSOR_X else wl.linears[li].o
    return to_bf16(normal_f32((m, width), 1.0, wl.wid, tensor, li, m))


def small_linear(h: int, o: int, r: int, m: int, seed: int, w_std: float = 0.02,
                 lora_std: float = 0.01):
    """A small seeded linear problem for parity tests: (W[o][h] f32, L1, L2, X, dY)."""
    w = torch.from_numpy(normal_f32((o, h), w_std, 100 + seed, TENSOR_W, h, o))
    l1 = to_bf16(normal_f32((h, r), lora_std, 100 + seed, TENSOR_L1, h, r)) if r else None
    l2 = to_bf16(normal_f32((r, o), lora_std, 100 + seed, TENSOR_L2, o, r)) if r else None
    x = to_bf16(normal_f32((m, h), 1.0, 100 + seed, TENSOR_X, m, h))
    dy = to_bf16(normal_f32((m, o), 1.0, 100 + seed, TENSOR_DY, m, o))
    return w, l1, l2, x, dy


def codec_chunk_f32(n: int, seed: int, std: float = 0.02, t_block_p: float = C4_T_BLOCK_P,
                    block: int = 64) -> np.ndarray:
    """float32 weights for the codec workload, generated on the host.

    N(0, std^2) entries; each aligned 64-entry block is, with probability
    ``t_block_p``, replaced by std * Student-t(4) draws (heavy-tailed blocks).
    """
    g = _rng(C4_CODEC_WID, TENSOR_W, 0, seed)
    w = g.standard_normal(size=n) * std
    nblk = (n + block - 1) // block
    heavy = np.flatnonzero(_rng(C4_CODEC_WID, TENSOR_MASK, 0, seed).random(size=nblk) < t_block_p)
    if heavy.size:
        t = _rng(C4_CODEC_WID, TENSOR_AUX, 0, seed).standard_t(4, size=(heavy.size, block)) * std
        idx = (heavy[:, None] * block + np.arange(block)[None, :]).ravel()
        keep = idx < n
        w[idx[keep]] = t.ravel()[keep]
    return w.astype(np.float32)


def codec_weights_device(n: int, seed: int, device, dtype=torch.bfloat16, std: float = 0.02,
                         t_block_p: float = C4_T_BLOCK_P, block: int = 64,
                         chunk: int = 1 << 28) -> torch.Tensor:
    """The codec workload generated directly on a GPU with PyTorch's seeded generator.

    Same distribution as :func:`codec_chunk_f32`; used where host generation of
    billions of entries would dominate run time.  Generated in chunks so the
    float32 temporaries stay small.
    """
    assert chunk % block == 0
    out = torch.empty(n, dtype=dtype, device=device)
    gen = torch.Generator(device=device)
    for ci, start in enumerate(range(0, n, chunk)):
        stop = min(n, start + chunk)
        m = stop - start
        gen.manual_seed(int(np.random.SeedSequence([C4_CODEC_WID, TENSOR_W, seed, ci]).generate_state(1)[0]))
        w = torch.randn(m, generator=gen, device=device, dtype=torch.float32) * std
        nblk = (m + block - 1) // block
        heavy = torch.rand(nblk, generator=gen, device=device) < t_block_p
        pad = nblk * block - m
        z = torch.randn(nblk, block, generator=gen, device=device, dtype=torch.float32)
        v = torch.randn(nblk, block, 4, generator=gen, device=device, dtype=torch.float32).square_().sum(-1)
        t = z / torch.sqrt(v / 4.0) * std
        w2 = torch.nn.functional.pad(w, (0, pad)).view(nblk, block)
        w2 = torch.where(heavy[:, None], t, w2).reshape(-1)[:m]
        out[start:stop] = w2.to(dtype)
        del w, z, v, t, w2, heavy
    return out
