"""CPU oracle of the W8A8 quantized-verification hot path (Quasar).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it.  It shares no code with the HIP
library or its Python binding, and it imports neither.

It is a plain, slow, step-by-step numpy rendering of what the verify step
computes, with every rounding written out, so a reader can check it against
the pages by eye:

* per-token symmetric int8 activation quantization, optionally after the
  smoothing multiply (``quant.quantize_act``);
* per-output-channel symmetric int8 weight quantization, optionally after the
  smoothing divide (``quant.quantize_weight``), and its 4-bit form for the
  W4A8 verifier (``quant.quantize_weight_int4``);
* the exact int8 x int8 -> int32 product (``gemm.int8_gemm``);
* the dequant epilogue to fp32 and bf16 (``gemm.dequant``);
* LM-head argmax and greedy acceptance (``accept``);
* stochastic verification at temperature T > 0: softmax of the dequantized
  logits, acceptance of each draft with its probability, residual or bonus
  sampling by inverse CDF (``sample``);
* the BF16 glue between linears: residual add, RMSNorm and SwiGLU before
  the next quantization (``glue``), and the verified block's causal,
  grouped-query attention over the KV cache (``attention``);
* the bf16 reference layer and the weight-traffic closed forms
  (``reference``).

Sources (all five pages summarise arXiv 2603.01399, "Quasar: Quantized
Self-Speculative Acceleration for Rapid Inference via Memory-Efficient
Verification"); cited below by site and section:

* [de] gist.science German summary, "Technische Zusammenfassung";
* [it] gist.science Italian summary, "Sommario tecnico";
* [fr] gist.science French summary, "Résumé technique";
* [zh] shd-paper.top Chinese summary, with the English abstract
  ("摘要（原文）");
* [ja] gist.science Japanese summary, "技術的サマリー".

Readings where the pages are silent (scale granularity, rounding mode, int8
range, dequant order, tie-break, acceptance rule) are stated in each
function's docstring.  Parity status: every function here is pinned by the
``-m "not gpu"`` oracle tests (closed forms, brute force, an independent
library cast, exhaustive small cases, invariants); none is unpinned.
"""
from .bf16 import bf16_to_f32, f32_to_bf16
from .quant import quantize_rows, quantize_act, quantize_weight, quantize_weight_int4
from .gemm import int8_gemm, dequant, w8a8_linear, INT32_MAX_K
from .accept import argmax_rows, greedy_accept, verify_accept
from .sample import exp_f32, fixed_weights, verify_sample
from .glue import residual_add, rmsnorm, silu_mul
from .attention import verify_attention, qk_norm_rope
from .reference import (bf16_reference_logits, w8a8_linear_bytes,
                        bf16_linear_bytes, weight_bytes_int8, weight_bytes_bf16)

__all__ = [
    "bf16_to_f32", "f32_to_bf16", "quantize_rows", "quantize_act",
    "quantize_weight", "int8_gemm", "dequant", "w8a8_linear", "INT32_MAX_K",
    "argmax_rows", "greedy_accept", "verify_accept", "bf16_reference_logits",
    "w8a8_linear_bytes", "bf16_linear_bytes", "weight_bytes_int8",
    "weight_bytes_bf16", "exp_f32", "fixed_weights", "verify_sample", "quantize_weight_int4",
    "residual_add", "rmsnorm", "silu_mul", "verify_attention", "qk_norm_rope",
]
