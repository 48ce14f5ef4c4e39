"""Pins for the oracle's int8 product and dequant epilogue.

* brute-force triple loop on tiny shapes (both routes);
* the f64 BLAS route equals the int64 route bit for bit on mid-size shapes;
* closed forms: all +127 x all -127 gives -16129*K; identity-like weights
  pick out columns;
* dequant: |y32 - acc*xs*ws| <= 3 ulp-ish relative (three fp32 roundings),
  checked in float64, with distinct per-row and per-column scales so that a
  swapped index fails; the bf16 output is the nearest-even bf16 of y32
  (checked through torch's cast);
* the W8A8 result against the unquantized product within the per-element
  quantization error bound;
* the smoothing identity Y = (W diag(s)^-1)(diag(s) X) in float64, and the
  smoothed W8A8 result within the same bound.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import (INT32_MAX_K, bf16_to_f32, dequant, int8_gemm, quantize_act,
                    quantize_weight, w8a8_linear)


def brute(xq, wq):
    M, K = xq.shape
    N = wq.shape[0]
    out = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        for n in range(N):
            s = 0
            for k in range(K):
                s += int(xq[m, k]) * int(wq[n, k])
            out[m, n] = s
    return out


def rand_i8(r, shape, full_range=True):
    lo = -128 if full_range else -127
    return r.integers(lo, 128, size=shape).astype(np.int8)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (5, 16, 64), (3, 7, 13), (5, 9, 48), (2, 3, 0)])
@pytest.mark.parametrize("route", ["int64", "f64"])
def test_brute_force_tiny(M, N, K, route):
    r = np.random.default_rng(M * 100 + N * 10 + K)
    xq = rand_i8(r, (M, K))
    wq = rand_i8(r, (N, K))
    got = int8_gemm(xq, wq, route=route)
    assert got.dtype == np.int32
    np.testing.assert_array_equal(got.astype(np.int64), brute(xq, wq))


def test_exhaustive_small_values():
    # every pair of int8 values in a K=1 product
    v = np.arange(-128, 128, dtype=np.int64)
    xq = v.astype(np.int8)[:, None]
    wq = v.astype(np.int8)[:, None]
    got = int8_gemm(xq, wq, route="int64").astype(np.int64)
    np.testing.assert_array_equal(got, np.outer(v, v))
    np.testing.assert_array_equal(int8_gemm(xq, wq, route="f64"), got.astype(np.int32))


@pytest.mark.parametrize("M,N,K", [(5, 512, 256), (8, 300, 4096), (16, 64, 25600)])
def test_f64_route_equals_int64_route(M, N, K):
    r = np.random.default_rng(K)
    xq = rand_i8(r, (M, K), full_range=False)
    wq = rand_i8(r, (N, K), full_range=False)
    np.testing.assert_array_equal(int8_gemm(xq, wq, "f64"), int8_gemm(xq, wq, "int64"))


@pytest.mark.parametrize("K", [64, 4096, 25600, INT32_MAX_K])
def test_closed_form_extremes(K):
    xq = np.full((2, K), 127, dtype=np.int8)
    wq = np.full((3, K), -127, dtype=np.int8)
    wq[1] = 127
    acc = int8_gemm(xq, wq)
    assert np.all(acc[:, 0] == -16129 * K) and np.all(acc[:, 1] == 16129 * K)


def test_k_bound():
    assert INT32_MAX_K == 133144
    assert 16129 * INT32_MAX_K <= 2**31 - 1 < 16129 * (INT32_MAX_K + 1)
    with pytest.raises(ValueError):
        int8_gemm(np.zeros((1, INT32_MAX_K + 1), np.int8), np.zeros((1, INT32_MAX_K + 1), np.int8))


def test_selector_weights_pick_columns():
    r = np.random.default_rng(3)
    xq = rand_i8(r, (5, 32))
    wq = np.zeros((32, 32), dtype=np.int8)
    perm = r.permutation(32)
    wq[np.arange(32), perm] = 1
    acc = int8_gemm(xq, wq)
    np.testing.assert_array_equal(acc, xq[:, perm].astype(np.int32))


def test_operand_orientation():
    # NT product: rows of xq against rows of wq; a transposed operand fails
    xq = np.array([[1, 2, 3]], dtype=np.int8)
    wq = np.array([[1, 0, 0], [0, 0, 2]], dtype=np.int8)
    np.testing.assert_array_equal(int8_gemm(xq, wq), [[1, 6]])


def test_dequant_closed_form_and_indexing():
    r = np.random.default_rng(4)
    M, N = 6, 37
    acc = r.integers(-400_000_000, 400_000_000, size=(M, N)).astype(np.int32)
    xs = (r.uniform(0.001, 0.2, size=M)).astype(np.float32)
    ws = (r.uniform(1e-5, 1e-3, size=N)).astype(np.float32)
    y32, y = dequant(acc, xs, ws)
    exact = acc.astype(np.float64) * xs.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]
    rel = np.abs(y32.astype(np.float64) - exact) / np.abs(exact)
    assert np.all(rel <= 3 * 2.0 ** -24 + 1e-15)
    # bf16 output is torch's nearest-even cast of y32
    t = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(y, t)


def test_dequant_exact_when_scales_are_powers_of_two():
    acc = np.array([[3, -5, 1 << 20]], dtype=np.int32)
    y32, _ = dequant(acc, np.array([0.25], np.float32), np.array([2.0, 0.5, 0.125], np.float32))
    np.testing.assert_array_equal(y32, np.array([[1.5, -0.625, float(1 << 15)]], np.float32))


def test_dequant_rounding_order():
    """(acc*xs)*ws and acc*(xs*ws) differ for some inputs; the oracle must
    follow the stated order: find such inputs and check which one it gives."""
    r = np.random.default_rng(44)
    found = 0
    for _ in range(2000):
        a = np.int32(r.integers(1, 2**30))
        xs = np.float32(r.uniform(0.001, 1))
        ws = np.float32(r.uniform(0.001, 1))
        left = np.float32(np.float32(np.float32(a) * xs) * ws)
        right = np.float32(np.float32(a) * np.float32(xs * ws))
        if left != right:
            y32, _ = dequant(np.array([[a]]), np.array([xs]), np.array([ws]))
            assert y32[0, 0] == left
            found += 1
    assert found > 10


def quant_error_bound(x32, w32, xs, ws):
    """Per-element bound on |W8A8 - exact product| from the round-trip bounds
    |x - qx*xs| <= ex and |w - qw*ws| <= ew (ex = xs*0.50003, ew = ws*0.50003):
    x*w - (qx*xs)(qw*ws) = qx*xs*dw + dx*qw*ws + dx*dw, so per k the error is
    at most |x|*ew + |w|*ex + 3*ex*ew; summed over k."""
    ex = xs.astype(np.float64) * 0.50003
    ew = ws.astype(np.float64) * 0.50003
    sx = np.abs(x32.astype(np.float64)).sum(axis=1)   # [M]
    sw = np.abs(w32.astype(np.float64)).sum(axis=1)   # [N]
    K = x32.shape[1]
    return sx[:, None] * ew[None, :] + ex[:, None] * sw[None, :] + 3 * K * ex[:, None] * ew[None, :]


@pytest.mark.parametrize("M,N,K", [(5, 512, 256), (5, 64, 4096)])
def test_w8a8_against_unquantized_product(M, N, K):
    bits = synth.activations_bf16(91, M, K, outliers=True)
    w = synth.weights_f32(91, N, K)
    xq, xs = quantize_act(bits)
    wq, ws = quantize_weight(w)
    acc, y32, _ = w8a8_linear(xq, xs, wq, ws)
    x = bf16_to_f32(bits)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    bound = quant_error_bound(x, w, xs, ws)
    err = np.abs(y32.astype(np.float64) - exact)
    assert np.all(err <= bound + 4 * 2.0 ** -24 * (np.abs(exact) + bound))
    # and the bound is not vacuous: typical error is far below it
    assert np.median(err / bound) < 0.1


def test_smoothing_identity_and_bound():
    """Y = (W diag(s)^-1)(diag(s) X) holds exactly up to fp64 rounding, and the
    smoothed W8A8 result stays within the quantization bound of W X."""
    M, N, K = 5, 96, 512
    bits = synth.activations_bf16(92, M, K, outliers=True)
    w = synth.weights_f32(92, N, K)
    s = synth.smoothing_vector(92, K)
    x = bf16_to_f32(bits).astype(np.float64)
    s64 = s.astype(np.float64)
    lhs = (w.astype(np.float64) / s64[None, :]) @ (x * s64[None, :]).T
    rhs = w.astype(np.float64) @ x.T
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))
    xq, xs = quantize_act(bits, smooth=s)
    wq, ws = quantize_weight(w, smooth=s)
    _, y32, _ = w8a8_linear(xq, xs, wq, ws)
    xsm = (bf16_to_f32(bits) * s[None, :]).astype(np.float32)
    wsm = (w / s[None, :]).astype(np.float32)
    bound = quant_error_bound(xsm, wsm, xs, ws)
    err = np.abs(y32.astype(np.float64) - rhs.T)
    assert np.all(err <= bound + 4 * 2.0 ** -24 * (np.abs(rhs.T) + bound) + 1e-9 * np.abs(rhs.T))


def test_smoothing_moves_outliers_to_weights():
    """With s = 1/|column max| on the outlier channels, the activation scale
    drops (the point of smoothing), and W8A8 error against W X shrinks."""
    M, N, K = 5, 128, 1024
    bits = synth.activations_bf16(93, M, K, outliers=True)
    x = bf16_to_f32(bits)
    w = synth.weights_f32(93, N, K)
    colmax = np.max(np.abs(x), axis=0).astype(np.float64)
    wmax = np.max(np.abs(w), axis=0).astype(np.float64)
    s = np.sqrt(wmax / colmax).astype(np.float32)  # alpha = 0.5 balance
    s = s / np.float32(np.median(s))
    xq0, xs0 = quantize_act(bits)
    xq1, xs1 = quantize_act(bits, smooth=s)
    wq0, ws0 = quantize_weight(w)
    wq1, ws1 = quantize_weight(w, smooth=s)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    _, y0, _ = w8a8_linear(xq0, xs0, wq0, ws0)
    _, y1, _ = w8a8_linear(xq1, xs1, wq1, ws1)
    e0 = np.sqrt(np.mean((y0 - ref) ** 2))
    e1 = np.sqrt(np.mean((y1 - ref) ** 2))
    assert e1 < e0
