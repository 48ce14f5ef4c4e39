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
