"""The BF16 glue between the verifier's W8A8 linears (oracle; test
infrastructure only): residual add + RMSNorm before the attention and MLP
linears, and the SwiGLU product before the down projection, each followed by
the per-token int8 quantization of the next linear's input.

The pages: the INT32 results are dequantized to BF16 before the non-linear
layers (normalisation, activation, softmax), which run in high precision
([de] §2 "De-Quantisierung"; [it] §2 pipeline, "Dequantizzazione"; [fr] §2
"Inférence en ligne": LayerNorm, GeLU; [ja] §2.2 item 3).  They name
LayerNorm and GeLU/Softmax generically; the Qwen3 shapes the workloads
follow use RMSNorm and SiLU-gated MLPs, so those are what is computed.

Readings (the pages give no formulas for these layers), following the
usual bf16 inference arithmetic:

* residual: h1 = bf16(fp32(h) + fp32(delta)) (the residual stream is bf16);
* RMSNorm: r = 1 / sqrt(mean_k h1_k^2 + eps), t_k = bf16(h1_k * r),
  n_k = bf16(t_k * gamma_k) (gamma bf16); here computed in float64, so the
  only rounding steps are the two bf16 roundings (an implementation in fp32
  differs from this by at most one bf16 step where h1_k * r sits next to a
  bf16 rounding boundary);
* SwiGLU: s_k = bf16(silu(g_k)), silu(g) = g / (1 + e^-g), in float64, then
  a_k = bf16(s_k * u_k);
* the next linear's input is then quantized by :func:`quant.quantize_act`
  on the bf16 values n (or a), optionally with the smoothing vector.
"""
import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16


def _f64_to_bf16_bits(v) -> np.ndarray:
    """Round float64 values directly to bf16: 8 significant bits, nearest,
    ties to even (no intermediate fp32 rounding).  Normal range only."""
    v = np.asarray(v, dtype=np.float64)
    # bf16 keeps 8 significant bits: round the float64 significand to 8 bits
    m, e = np.frexp(v)                         # v = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return f32_to_bf16(r.astype(np.float32))   # r is exactly representable in bf16


def residual_add(h_bits, delta_bits=None) -> np.ndarray:
    """bf16 bits of bf16(fp32(h) + fp32(delta)) (h itself without delta)."""
    h = bf16_to_f32(h_bits)
    if delta_bits is None:
        return np.asarray(h_bits, dtype=np.uint16).copy()
    s = (h + bf16_to_f32(delta_bits)).astype(np.float32)
    return f32_to_bf16(s)


def rmsnorm(h1_bits, gamma_bits, eps: float) -> np.ndarray:
    """bf16 bits of n = bf16(bf16(h1 * r) * gamma), r = 1/sqrt(mean(h1^2) + eps),
    per row of h1 [M][D], in float64."""
    h1 = bf16_to_f32(h1_bits).astype(np.float64)
    g = bf16_to_f32(gamma_bits).astype(np.float64)
    if h1.ndim != 2 or g.shape != (h1.shape[1],):
        raise ValueError("rmsnorm expects h1 [M][D] and gamma [D]")
    var = np.mean(h1 * h1, axis=1, keepdims=True)
    r = 1.0 / np.sqrt(var + float(eps))
    t = bf16_to_f32(_f64_to_bf16_bits(h1 * r)).astype(np.float64)
    return _f64_to_bf16_bits(t * g[None, :])


def silu_mul(gate_bits, up_bits) -> np.ndarray:
    """bf16 bits of a = bf16(bf16(silu(g)) * u), silu(g) = g / (1 + e^-g), in
    float64."""
    g = bf16_to_f32(gate_bits).astype(np.float64)
    u = bf16_to_f32(up_bits).astype(np.float64)
    with np.errstate(over="ignore"):
        s = g / (1.0 + np.exp(-g))
    sb = bf16_to_f32(_f64_to_bf16_bits(s)).astype(np.float64)
    return _f64_to_bf16_bits(sb * u)
