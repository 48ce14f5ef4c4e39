"""bf16 <-> fp32 conversions (oracle; test infrastructure only).

The verifier keeps its inputs and its dequantized outputs in BF16 ([ja]
§2.2 item 3, online inference; [it] §2 pipeline, "Dequantizzazione").  A
bf16 number is the upper 16 bits of an IEEE binary32 word.
"""
import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32.

    The bf16 pattern is the top half of the fp32 word and the low half is
    zero, so the widening is exact."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x) -> np.ndarray:
    """Narrow float32 to bf16 bit patterns (uint16), round to nearest with
    ties to even.

    Dropping the low 16 bits after adding 0x7FFF plus the lowest kept bit
    rounds the magnitude to nearest-even: below half drops, above half
    carries, exactly half carries only when the kept part is odd.  Values
    beyond the largest finite bf16 round to infinity (the carry runs into
    the exponent).  NaN stays NaN (quiet bit set, sign kept)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    keep_lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + keep_lsb) >> 16
    quiet = (u >> 16) | 0x40
    return np.where(is_nan, quiet, rounded).astype(np.uint16)
