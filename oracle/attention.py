"""Attention of the verified block over the KV cache (oracle; test
infrastructure only).

The pages keep the non-linear parts of the verifier, softmax among them, in
high precision after the dequant step ([de] §2 "De-Quantisierung"; [it] §2
pipeline; [ja] §2.2 item 3).  In one verification step the T = G + 1 new
positions of each sequence are checked together, so each of them attends
to the cached context and to the new positions up to and including itself.

Reading (the pages give no attention formula; this is the usual causal,
grouped-query form of the Qwen3 shapes):

* q [B][T][Hq][Dh], the cache k, v [B][Hkv][Lmax][Dh], all bf16; the first
  L_b positions of sequence b's cache are valid and the last T of them are
  the verified block's own keys and values;
* query i of sequence b, head h reads kv head h // (Hq / Hkv) and the keys
  j <= L_b - T + i;
* o = softmax(q . k_j / sqrt(Dh)) . v, computed here in float64, rounded
  once to bf16 (nearest, ties to even).
"""
import numpy as np

from .bf16 import bf16_to_f32
from .glue import _f64_to_bf16_bits


def verify_attention(q_bits, k_bits, v_bits, lengths) -> np.ndarray:
    """bf16 bits of the attention output [B][T][Hq][Dh] (see module doc)."""
    q = bf16_to_f32(q_bits).astype(np.float64)
    k = bf16_to_f32(k_bits).astype(np.float64)
    v = bf16_to_f32(v_bits).astype(np.float64)
    B, T, Hq, Dh = q.shape
    _, Hkv, Lmax, _ = k.shape
    if Hq % Hkv != 0 or k.shape != v.shape or k.shape[0] != B or k.shape[3] != Dh:
        raise ValueError("shape mismatch")
    lengths = np.asarray(lengths, dtype=np.int64)
    if np.any(lengths < T) or np.any(lengths > Lmax):
        raise ValueError("each length must be in [T, Lmax]")
    group = Hq // Hkv
    out = np.empty((B, T, Hq, Dh), dtype=np.float64)
    scale = 1.0 / np.sqrt(Dh)
    for b in range(B):
        for i in range(T):
            last = int(lengths[b]) - T + i          # inclusive
            for h in range(Hq):
                kh = h // group
                s = k[b, kh, :last + 1] @ q[b, i, h] * scale
                p = np.exp(s - s.max())
                p /= p.sum()
                out[b, i, h] = p @ v[b, kh, :last + 1]
    return _f64_to_bf16_bits(out)


def qk_norm_rope(qkv_bits, B, T, Hq, Hkv, q_gamma_bits, k_gamma_bits, eps, start, base):
    """The steps between the [q;k;v] linear and attention, per token row
    (b, i) of ``qkv [B*T][(Hq + 2 Hkv) * 128]`` (bf16; heads of q, then k,
    then v, 128 columns each):

    * per-head RMSNorm of q and k over their 128 dims with bf16 gammas:
      n = bf16(bf16(x * r) * gamma), r = 1/sqrt(mean(x^2) + eps);
    * rotary position embedding at position p = start[b] + i, rotating dim
      pairs (d, d + 64), d < 64, by the angle a = fp32(fp32(p) * f_d) with
      f_d = fp32(base^(-d/64)) (the fp32 angle of bf16/fp32 inference: at
      positions near 1e5 its rounding moves the angle by up to ~4e-3, which
      this reproduces rather than corrects): (x1, x2) -> (x1 cos a - x2 sin a,
      x2 cos a + x1 sin a), cos and sin in float64, rounded to bf16;
    * v unchanged.

    Returns bf16 bits ``q [B][T][Hq][128]``, ``k [B][T][Hkv][128]``,
    ``v [B][T][Hkv][128]``, in float64 with direct bf16 rounding (Qwen3's
    q/k norms and its rotate-half RoPE; the pages do not describe the
    attention block)."""
    from .glue import rmsnorm
    x = np.asarray(qkv_bits, dtype=np.uint16).reshape(B, T, Hq + 2 * Hkv, 128)
    qg = np.asarray(q_gamma_bits, dtype=np.uint16)
    kg = np.asarray(k_gamma_bits, dtype=np.uint16)
    qn = rmsnorm(x[:, :, :Hq].reshape(-1, 128), qg, eps).reshape(B, T, Hq, 128)
    kn = rmsnorm(x[:, :, Hq:Hq + Hkv].reshape(-1, 128), kg, eps).reshape(B, T, Hkv, 128)
    v = x[:, :, Hq + Hkv:].copy()
    d = np.arange(64, dtype=np.float64)
    inv_freq = (float(base) ** (-d / 64.0)).astype(np.float32)
    pos = (np.asarray(start, dtype=np.int64)[:, None] + np.arange(T)[None, :]).astype(np.float32)
    ang = (pos[:, :, None] * inv_freq[None, None, :]).astype(np.float32)   # B T 64, fp32 product
    cos, sin = np.cos(ang.astype(np.float64)), np.sin(ang.astype(np.float64))

    def rope(h_bits):
        h = bf16_to_f32(h_bits).astype(np.float64)
        x1, x2 = h[..., :64], h[..., 64:]
        c, s = cos[:, :, None, :], sin[:, :, None, :]
        out = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
        return _f64_to_bf16_bits(out)

    return rope(qn), rope(kn), v
