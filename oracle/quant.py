"""Symmetric int8 quantization of activations and weights (oracle; test
infrastructure only).

What the pages fix:
* W8A8: weights and activations both in 8 bits ([de] §2 "Kernidee";
  [it] §2 "Concetto Chiave"; [ja] §2.1);
* symmetric uniform quantization ([it] §2 "Componenti Tecnici" 1);
* weights are smoothed and quantized to INT8 offline, ahead of inference
  ([it] §2 pipeline, "Preparazione Offline"; [ja] §2.2 item 2);
* activations arrive in BF16 and are scaled by the smoothing factor s and
  converted to INT8 dynamically, at run time ([de] §2 "Online-Prozess";
  [it] §2 pipeline, "Inferenza Online"; [ja] §2.2 item 3);
* the smoothing transform Y = (W diag(s)^-1)(diag(s) X) ([ja] §2.2 item 1),
  i.e. activations are multiplied by s per input channel and weights divided
  by it.

Readings where the pages are silent (each is a plain textbook choice):
* granularity: one scale per activation row (token, "dynamic") and one per
  weight row (output channel);
* int8 range [-127, 127] (symmetric; -128 is never produced);
* scale = amax / 127 and the quantizer multiplies by inv = 127 / amax, both
  correctly rounded fp32 divisions computed once per row;
* q = clip(round_half_even(fp32(v * inv)), -127, 127);
* amax == 0 gives scale = inv = 0 and q = 0;
* an element equal to zero always quantizes to 0 (this only matters when
  127 / amax overflows fp32, i.e. amax < 127 / FLT_MAX, where 0 * inf would
  otherwise be NaN); nonzero elements of such a row saturate to +-127;
* inputs must be finite (non-finite input raises).
"""
import numpy as np

from .bf16 import bf16_to_f32



def quantize_rows(v, qmax: int = 127) -> tuple:
    """Quantize each row of a finite fp32 matrix ``v[R][C]`` to integer codes
    in [-qmax, qmax] (127 for int8; 7 for the int4 weights of W4A8).

    Returns ``(q int8[R][C], scale float32[R])`` with, per row r:
      amax  = max_c |v[r, c]|                       (exact)
      scale = fp32(amax / qmax)
      inv   = fp32(qmax / amax)                     (0 when amax == 0)
      q     = clip(rint(fp32(v * inv)), -qmax, qmax) (0 where v == 0)
    """
    v = np.asarray(v, dtype=np.float32)
    if v.ndim != 2:
        raise ValueError("quantize_rows expects a 2-D array")
    if not np.all(np.isfinite(v)):
        raise ValueError("quantize_rows: input must be finite")
    if qmax not in (127, 7):
        raise ValueError("qmax must be 127 (int8) or 7 (int4)")
    fq = np.float32(qmax)
    R = v.shape[0]
    if v.shape[1] == 0:
        return np.zeros(v.shape, dtype=np.int8), np.zeros(R, dtype=np.float32)
    amax = np.max(np.abs(v), axis=1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1.0))
    with np.errstate(over="ignore", divide="ignore"):
        scale = np.where(nz, safe / fq, np.float32(0.0)).astype(np.float32)
        inv = np.where(nz, fq / safe, np.float32(0.0)).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        prod = (v * inv[:, None]).astype(np.float32)
        q = np.rint(prod)
    q = np.where(v == 0, np.float32(0.0), q)
    q = np.clip(q, -qmax, qmax)
    return q.astype(np.int8), scale


def quantize_act(x_bf16_bits, smooth=None) -> tuple:
    """Per-token activation quantization of bf16 input ``x[M][K]``.

    x' = fp32(x) * s[k] (one fp32 multiply per element) when the smoothing
    vector ``smooth`` (positive, finite, length K) is given, else x' = fp32(x);
    then :func:`quantize_rows` on x'.  Returns ``(xq int8[M][K],
    x_scale float32[M])``."""
    x = bf16_to_f32(x_bf16_bits)
    if x.ndim != 2:
        raise ValueError("quantize_act expects [M][K]")
    if smooth is not None:
        s = np.asarray(smooth, dtype=np.float32)
        if s.shape != (x.shape[1],):
            raise ValueError("smooth must have length K")
        x = (x * s[None, :]).astype(np.float32)
    return quantize_rows(x)


def quantize_weight(w_f32, smooth=None) -> tuple:
    """Per-output-channel weight quantization of fp32 ``W[N][K]``.

    w' = fp32(W[n, k] / s[k]) (one correctly rounded fp32 division) when
    ``smooth`` is given, else w' = W; then :func:`quantize_rows` on w'.
    Returns ``(wq int8[N][K], w_scale float32[N])``."""
    w = np.asarray(w_f32, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("quantize_weight expects [N][K]")
    if smooth is not None:
        s = np.asarray(smooth, dtype=np.float32)
        if s.shape != (w.shape[1],):
            raise ValueError("smooth must have length K")
        w = (w / s[None, :]).astype(np.float32)
    return quantize_rows(w)


def quantize_weight_int4(w_f32, smooth=None) -> tuple:
    """Per-output-channel symmetric int4 quantization of fp32 ``W[N][K]``
    (the W4A8 verifier's weights): :func:`quantize_weight` with codes in
    [-7, 7] and scale = fp32(amax / 7).  Returns ``(wq int8[N][K] holding the
    int4 codes, w_scale float32[N])``.

    The pages name lower-bit verifiers, INT4 among them, as explored or as
    the next step ([zh] 关键设计; [it] §5; [ja] §5); they give no scheme.
    Reading: the int8 scheme above with 4-bit codes, one scale per output
    channel, symmetric, -8 never produced; the product with int8
    activations is then the same exact integer contraction."""
    w = np.asarray(w_f32, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("quantize_weight_int4 expects [N][K]")
    if smooth is not None:
        s = np.asarray(smooth, dtype=np.float32)
        if s.shape != (w.shape[1],):
            raise ValueError("smooth must have length K")
        w = (w / s[None, :]).astype(np.float32)
    return quantize_rows(w, qmax=7)
