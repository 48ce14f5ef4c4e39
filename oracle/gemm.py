"""INT8 product with INT32 accumulation and the dequant epilogue (oracle;
test infrastructure only).

The pages: the matrix product runs on INT8 units with the result
accumulated in INT32, then dequantized back to high precision (BF16) before
the nonlinear layers ([ja] §2.2 item 3; [de] §2 "Online-Prozess" and
"De-Quantisierung"; [it] §2 pipeline, "Calcolo" / "Dequantizzazione"; [fr]
§2 pipeline technique).

Readings (pages silent): the product is "NT" — both operands are stored with
K contiguous (activations ``[M][K]``, weights ``[N][K]`` in nn.Linear order);
dequant is y32 = fp32(fp32(fp32(acc) * x_scale[m]) * w_scale[n]) — the int32
to fp32 conversion and two multiplies, each correctly rounded, in this
order, with no fused multiply-add — and y = bf16_rne(y32).
"""
import numpy as np

from .bf16 import f32_to_bf16

# Largest K for which |sum_k q_x q_w| <= 127*127*K always fits in int32.
INT32_MAX_K = (2**31 - 1) // (127 * 127)


def int8_gemm(xq, wq, route: str = "f64") -> np.ndarray:
    """Exact ``acc[m, n] = sum_k xq[m, k] * wq[n, k]`` as int32.

    ``route="int64"`` multiplies in int64; ``route="f64"`` uses a float64
    matrix product, which is exact here because every partial sum is an
    integer of magnitude <= 127*127*K < 2**53 (any summation order).  Both
    routes are checked against each other and against a brute-force loop."""
    xq = np.asarray(xq)
    wq = np.asarray(wq)
    if xq.dtype != np.int8 or wq.dtype != np.int8:
        raise TypeError("int8_gemm expects int8 operands")
    if xq.ndim != 2 or wq.ndim != 2 or xq.shape[1] != wq.shape[1]:
        raise ValueError("int8_gemm expects xq[M][K], wq[N][K]")
    K = xq.shape[1]
    if K > INT32_MAX_K:
        raise ValueError("K too large for an exact int32 accumulator")
    if route == "int64":
        acc = xq.astype(np.int64) @ wq.astype(np.int64).T
    elif route == "f64":
        accf = xq.astype(np.float64) @ wq.astype(np.float64).T
        acc = accf.astype(np.int64)
        if not np.array_equal(acc.astype(np.float64), accf):
            raise AssertionError("f64 route produced a non-integer")
    else:
        raise ValueError(route)
    if acc.size and np.max(np.abs(acc)) > 2**31 - 1:
        raise AssertionError("accumulator exceeds int32")
    return acc.astype(np.int32)


def dequant(acc, x_scale, w_scale) -> tuple:
    """``y32[m, n] = fp32(fp32(fp32(acc[m, n]) * x_scale[m]) * w_scale[n])``
    and ``y = bf16_rne(y32)`` (returned as uint16 bit patterns)."""
    acc = np.asarray(acc, dtype=np.int32)
    xs = np.asarray(x_scale, dtype=np.float32)
    ws = np.asarray(w_scale, dtype=np.float32)
    a32 = acc.astype(np.float32)
    t = (a32 * xs[:, None]).astype(np.float32)
    y32 = (t * ws[None, :]).astype(np.float32)
    return y32, f32_to_bf16(y32)


def w8a8_linear(xq, x_scale, wq, w_scale, route: str = "f64") -> tuple:
    """One W8A8 linear: returns ``(acc int32, y32 float32, y bf16 bits)``."""
    acc = int8_gemm(xq, wq, route=route)
    y32, y = dequant(acc, x_scale, w_scale)
    return acc, y32, y
