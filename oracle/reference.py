"""The BF16 reference layer and weight-traffic closed forms (oracle; test
infrastructure only).

The pages: standard verification runs the target in BF16 ([de] §1
"Ursache"; [ja] §1); INT8 weights halve the memory traffic ([zh] abstract;
[de] §2 "Vorteil"; [it] §3; [ja] §2.1); verification latency is weight bytes
over bandwidth, M*2B/BW for BF16 against M*1B/BW for INT8 ([de] §3 item 4;
[ja] §2.3).
"""
import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16


def bf16_reference_logits(x_bf16_bits, w_f32) -> np.ndarray:
    """The BF16 verifier's linear: ``ref[m, n] = sum_k x[m, k] * bf16(W)[n, k]``
    with x the bf16 activations and W rounded to bf16 (nearest-even); the
    products and the sum are taken in float64."""
    x = bf16_to_f32(x_bf16_bits).astype(np.float64)
    wb = bf16_to_f32(f32_to_bf16(w_f32)).astype(np.float64)
    return x @ wb.T


def weight_bytes_int8(N: int, K: int) -> int:
    """Bytes of an int8 per-output-channel weight: N*K codes + N fp32 scales."""
    return N * K + 4 * N


def weight_bytes_bf16(N: int, K: int) -> int:
    """Bytes of a bf16 weight."""
    return 2 * N * K


def w8a8_linear_bytes(M: int, N: int, K: int, y_bf16=True, y_f32=False,
                      acc=False) -> int:
    """Algorithmic HBM bytes of one W8A8 linear: int8 weight + scales, int8
    activations + per-token scales, and each requested output."""
    b = weight_bytes_int8(N, K) + M * K + 4 * M
    b += (2 * M * N if y_bf16 else 0) + (4 * M * N if y_f32 else 0) + (4 * M * N if acc else 0)
    return b


def bf16_linear_bytes(M: int, N: int, K: int, y_bf16=True, y_f32=False) -> int:
    """Algorithmic HBM bytes of the same linear in BF16: bf16 weight, bf16
    activations, requested outputs."""
    return (weight_bytes_bf16(N, K) + 2 * M * K + (2 * M * N if y_bf16 else 0)
            + (4 * M * N if y_f32 else 0))
