"""Pins of the oracle's int4 weight quantizer (W4A8; oracle/quant.py,
quantize_weight_int4) against what arithmetic fixes: hand-derived ties, the
round-trip bound, saturation at the row maximum, the identity on integer
rows, the approximation bound of the W4A8 product against the unquantized
one, and its expected ratio to the W8A8 error."""
import numpy as np
import pytest

import oracle
from oracle.quant import quantize_rows, quantize_weight_int4

RNG = np.random.default_rng(404)


# rows whose products v * inv are exact, so the half-even rule decides
# (amax = 14 -> scale 2, inv 0.5; amax = 7 -> scale 1, inv 1)
WORKED = [
    ([14.0, 1.0, 3.0, -5.0, 0.0, 7.0], [7, 0, 2, -2, 0, 4], 2.0),
    ([7.0, 0.5, 1.5, 2.5, -3.5, -0.5], [7, 0, 2, 2, -4, 0], 1.0),
    ([-7.0, 6.5, 5.5, 4.5], [-7, 6, 6, 4], 1.0),
    ([28.0, 2.0, 6.0, 10.0, -14.0], [7, 0, 2, 2, -4], 4.0),   # inv = 0.25: 0.5, 1.5, 2.5, -3.5
    ([0.0, 0.0, 0.0], [0, 0, 0], 0.0),
]


@pytest.mark.parametrize("row,codes,scale", WORKED)
def test_worked_ties(row, codes, scale):
    q, s = quantize_weight_int4(np.array([row], dtype=np.float32))
    np.testing.assert_array_equal(q[0], np.array(codes, dtype=np.int8))
    assert s[0] == np.float32(scale)


def test_round_trip_bound_and_range():
    w = (RNG.standard_normal((300, 1000)) * 0.02).astype(np.float32)
    w[:, 17] *= 30                                      # an outlier channel
    q, s = quantize_weight_int4(w)
    assert q.min() >= -7 and q.max() <= 7
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 3e-5))
    # the largest magnitude of each row saturates
    idx = np.argmax(np.abs(w), axis=1)
    np.testing.assert_array_equal(np.abs(q[np.arange(300), idx]), 7)
    # signs are kept (or the code is 0)
    assert np.all((np.sign(q) == np.sign(w)) | (q == 0))


def test_integer_rows_are_their_own_codes():
    base = RNG.integers(-7, 8, size=(50, 64)).astype(np.float32)
    base[:, 0] = 7.0                                    # amax = 7: scale = inv = 1
    q, s = quantize_weight_int4(base)
    np.testing.assert_array_equal(q, base.astype(np.int8))
    np.testing.assert_array_equal(s, np.ones(50, dtype=np.float32))


def test_power_of_two_rescaling_and_smoothing():
    w = (RNG.standard_normal((20, 256)) * 0.05).astype(np.float32)
    q1, s1 = quantize_weight_int4(w)
    q2, s2 = quantize_weight_int4((w * np.float32(8)).astype(np.float32))
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s2, (s1 * np.float32(8)).astype(np.float32))
    sm = np.full(256, 4.0, dtype=np.float32)
    q3, s3 = quantize_weight_int4(w, smooth=sm)
    np.testing.assert_array_equal(q3, q1)
    np.testing.assert_array_equal(s3, (s1 / np.float32(4)).astype(np.float32))


def test_int8_default_is_unchanged():
    w = (RNG.standard_normal((10, 128))).astype(np.float32)
    np.testing.assert_array_equal(quantize_rows(w)[0], oracle.quantize_weight(w)[0])
    with pytest.raises(ValueError):
        quantize_rows(w, qmax=15)


def test_w4a8_product_bound_and_error_ratio():
    M, N, K = 5, 64, 1024
    x = (RNG.standard_normal((M, K))).astype(np.float32)
    bits = oracle.f32_to_bf16(x)
    xf = oracle.bf16_to_f32(bits).astype(np.float64)
    w = (RNG.standard_normal((N, K)) * 0.02).astype(np.float32)
    xq, xs = oracle.quantize_act(bits)
    q4, s4 = quantize_weight_int4(w)
    q8, s8 = oracle.quantize_weight(w)
    _, y4, _ = oracle.w8a8_linear(xq, xs, q4, s4)
    _, y8, _ = oracle.w8a8_linear(xq, xs, q8, s8)
    exact = xf @ w.astype(np.float64).T
    ex = (xs.astype(np.float64) * 0.50003)[:, None]              # per row of x
    ew = (s4.astype(np.float64) * 0.50003)[None, :]              # per channel
    bound = (np.abs(xf) @ np.ones((K, N))) * ew + ex * (np.ones((M, K)) @ np.abs(w.astype(np.float64)).T) \
        + K * ex * ew
    assert np.all(np.abs(y4 - exact) <= bound * 1.0001 + 1e-6)
    e4 = np.sqrt(np.mean((y4 - exact) ** 2))
    e8 = np.sqrt(np.mean((y8 - exact) ** 2))
    # 4-bit weight steps are 127/7 ~ 18x coarser; the activation error is shared
    assert 8 < e4 / e8 < 25
