"""CPU oracle for the QLoRA NF4 linear layer — TEST INFRASTRUCTURE ONLY.

A plain, slow, deliberately unoptimised restatement of what the QLoRA pages
describe: the NF4 codebook, blockwise quantization, double quantization of the
block scales, dequantization, and the LoRA linear layer's forward and backward
passes in float64.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product library
(``bit_quantized_fine_nf4_amd``) never imports it, and it never imports the
product: the two share no code, tables or constants.

Pages cited (by title and section):
  [TL]  "QLoRA: a memory budget is more than weight precision" (Token Lab)
  [MC]  "QLoRA: Efficient Finetuning of Quantized LLMs" (Michał Chromiak's blog)
  [SV]  "Chapter 1: What is QLoRA?" (SkillVerse course notes)
  [GO]  "QLoRA: the paper that put large-model fine-tuning on a desk" (Good Omens blog)
  [TT]  "QLoRA in LLMs" (TensorTonic)

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, worked examples printed on the pages, brute force on tiny
inputs, finite differences and invariants); none is "parity unpinned".
"""
from .nf4 import (  # noqa: F401
    NF4_DELTA, nf4_levels, nf4_levels_f64, nf4_midpoints, encode, quantize, quantize_bf16,
    int8_absmax_quantize, exact_mean_f32, double_quant, scale_reconstruct, dequantize,
    dequantize_no_dq, f32_to_bf16_bits, bf16_bits_to_f32, unpack_codes,
)
from .linear import linear_fwd, linear_bwd, dequantized_weight, merged_weight  # noqa: F401
from .ledger import storage_bits_per_weight, storage_bytes, lora_param_count  # noqa: F401
from .optim import adamw_step  # noqa: F401
from .glue import sigmoid, silu_gate_fwd, silu_gate_bwd, grad_sum  # noqa: F401
from . import codebooks  # noqa: F401
