"""Pins for the oracle's symmetric int8 quantizers.

* worked cases from tests/golden/quant_worked_cases.txt (hand-derived ties);
* scale and inv are the correctly rounded fp32 quotients, checked with exact
  rational arithmetic (fractions), not with the oracle's own formula;
* the round-trip bound |x' - q*scale| <= scale*(0.5 + 3e-5), in float64;
* invariants: range, saturation at the row's largest magnitude, sign, exact
  power-of-two rescaling, permutation equivariance, row independence;
* the smoothing path against the plain path where smoothing is exact.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import bf16_to_f32, quantize_act, quantize_rows, quantize_weight

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_worked_cases.txt")


def load_worked_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            xs, qs, sc = (p.strip() for p in line.split(";"))
            x = np.array([float(v) for v in xs.split(",")], dtype=np.float32)
            q = np.array([int(v) for v in qs.split(",")], dtype=np.int8)
            cases.append((x, q, float(sc)))
    return cases


WORKED = load_worked_cases()


def test_worked_cases_present():
    assert len(WORKED) >= 15


@pytest.mark.parametrize("x,q,scale", WORKED)
def test_worked_cases(x, q, scale):
    got_q, got_s = quantize_rows(x[None, :])
    np.testing.assert_array_equal(got_q[0], q)
    assert float(got_s[0]) == scale


@pytest.mark.parametrize("x,q,scale", WORKED)
def test_worked_cases_through_bf16_and_weight_paths(x, q, scale):
    from synth import to_bf16_bits
    bits = to_bf16_bits(x[None, :])
    assert np.array_equal(bf16_to_f32(bits)[0], x)  # fixture values are bf16-exact
    qa, sa = quantize_act(bits)
    np.testing.assert_array_equal(qa[0], q)
    qw, sw = quantize_weight(x[None, :])
    np.testing.assert_array_equal(qw[0], q)
    assert float(sa[0]) == float(sw[0]) == scale


def _nearest_f32(fr: Fraction) -> float:
    """Correctly rounded fp32 of a positive rational, by exhaustive neighbour
    search around float64's estimate."""
    est = np.float32(float(fr))
    cands = [est, np.nextafter(est, np.float32(np.inf)), np.nextafter(est, np.float32(0))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c, dtype=np.float32).view(np.uint32)) & 1))
    return float(best)


def test_scale_is_correctly_rounded_quotient():
    r = np.random.default_rng(5)
    x = r.standard_normal((400, 64)).astype(np.float32) * np.float32(3.0)
    _, scale = quantize_rows(x)
    amax = np.max(np.abs(x), axis=1)
    for a, s in zip(amax, scale):
        assert float(s) == _nearest_f32(Fraction(float(a)) / 127)


def test_inv_is_correctly_rounded_quotient():
    # q at an element that is exactly amax/2 reveals inv: q = rint(fl(amax/2 * inv))
    # and amax*inv rounds to 127 only if inv is within a few ulps of 127/amax
    r = np.random.default_rng(6)
    for _ in range(200):
        a = np.float32(abs(r.standard_normal()) + 0.1)
        row = np.array([a, a / np.float32(2), -a], dtype=np.float32)
        q, _ = quantize_rows(row[None, :])
        assert q[0, 0] == 127 and q[0, 2] == -127
        assert q[0, 1] in (63, 64)


def roundtrip_ok(x, q, scale):
    x64 = x.astype(np.float64)
    rec = q.astype(np.float64) * scale.astype(np.float64)[:, None]
    bound = scale.astype(np.float64)[:, None] * (0.5 + 3e-5)
    return np.all(np.abs(x64 - rec) <= bound)


@pytest.mark.parametrize("shape,spread", [((64, 256), 1.0), ((16, 4096), 1.0),
                                          ((32, 1000), 1e-20), ((8, 512), 1e30)])
def test_roundtrip_bound(shape, spread):
    r = np.random.default_rng(7)
    x = (r.standard_normal(shape) * spread).astype(np.float32)
    q, s = quantize_rows(x)
    assert roundtrip_ok(x, q, s)


def test_roundtrip_bound_with_outlier_activations():
    bits = synth.activations_bf16(99, 5, 4096, outliers=True)
    q, s = quantize_act(bits)
    assert roundtrip_ok(bf16_to_f32(bits), q, s)


def test_invariants():
    r = np.random.default_rng(8)
    x = r.standard_normal((50, 333)).astype(np.float32)
    x[3, 10] = 0.0
    x[4] = -x[4]
    q, s = quantize_rows(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert q.min() >= -127 and q.max() <= 127
    # the largest magnitude of each row saturates to +-127 with its sign
    j = np.argmax(np.abs(x), axis=1)
    rows = np.arange(x.shape[0])
    np.testing.assert_array_equal(q[rows, j], np.where(x[rows, j] > 0, 127, -127))
    # sign(q) is sign(x) or 0
    assert np.all((np.sign(q) == np.sign(x)) | (q == 0))
    # negating the input negates the output exactly (symmetric quantizer)
    qn, sn = quantize_rows(-x)
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(sn, s)


@pytest.mark.parametrize("j", [-40, -3, -1, 1, 5, 60])
def test_power_of_two_rescaling_is_exact(j):
    r = np.random.default_rng(9)
    x = r.standard_normal((20, 128)).astype(np.float32)
    q, s = quantize_rows(x)
    q2, s2 = quantize_rows((x * np.float32(2.0 ** j)).astype(np.float32))
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, (s * np.float32(2.0 ** j)).astype(np.float32))


def test_permutation_and_row_independence():
    r = np.random.default_rng(10)
    x = r.standard_normal((12, 200)).astype(np.float32)
    q, s = quantize_rows(x)
    perm = r.permutation(200)
    qp, sp = quantize_rows(x[:, perm])
    np.testing.assert_array_equal(qp, q[:, perm])
    np.testing.assert_array_equal(sp, s)
    for i in range(12):
        qi, si = quantize_rows(x[i:i + 1])
        np.testing.assert_array_equal(qi[0], q[i])
        assert si[0] == s[i]


def test_zero_rows_and_tiny_rows():
    x = np.zeros((3, 40), dtype=np.float32)
    x[1, 5] = -0.0
    # amax below 127/FLT_MAX: inv overflows; zeros stay 0, nonzeros saturate
    x[2, :] = 0
    x[2, 7] = np.float32(1e-38)
    x[2, 8] = np.float32(-1e-39)
    q, s = quantize_rows(x)
    assert np.all(q[:2] == 0) and s[0] == 0 and s[1] == 0
    assert q[2, 7] == 127 and q[2, 8] == -127
    assert np.count_nonzero(q[2]) == 2
    assert s[2] > 0


def test_non_finite_raises():
    x = np.ones((2, 4), dtype=np.float32)
    x[1, 2] = np.inf
    with pytest.raises(ValueError):
        quantize_rows(x)


def test_smoothing_by_powers_of_two_is_exact():
    """With s = 2^e per channel, x*s is exact in fp32, so quantize_act(x, s)
    equals the plain quantizer applied to the exactly scaled input; dividing
    weights by the same s is exact too."""
    r = np.random.default_rng(12)
    K = 256
    e = r.integers(-3, 4, size=K)
    s = (2.0 ** e).astype(np.float32)
    bits = synth.activations_bf16(98, 5, K)
    x = bf16_to_f32(bits)
    q1, s1 = quantize_act(bits, smooth=s)
    q2, s2 = quantize_rows((x.astype(np.float64) * s.astype(np.float64)).astype(np.float32))
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)
    w = r.standard_normal((7, K)).astype(np.float32)
    qw1, sw1 = quantize_weight(w, smooth=s)
    qw2, sw2 = quantize_rows((w.astype(np.float64) / s.astype(np.float64)).astype(np.float32))
    np.testing.assert_array_equal(qw1, qw2)
    np.testing.assert_array_equal(sw1, sw2)


def test_smoothing_general_vector_roundtrip():
    s = synth.smoothing_vector(97, 512)
    bits = synth.activations_bf16(97, 6, 512, outliers=True)
    q, sc = quantize_act(bits, smooth=s)
    xs = (bf16_to_f32(bits) * s[None, :]).astype(np.float32)
    assert roundtrip_ok(xs, q, sc)
