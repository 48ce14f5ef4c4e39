"""Pins of the oracle's BF16 glue (oracle/glue.py): direct float64 -> bf16
rounding on hand-derived ties and a double-rounding trap, the residual add
against torch's CPU bf16 addition, RMSNorm on closed-form rows and its scale
invariance, SwiGLU against scipy's logistic function and its limits."""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from oracle import glue

RNG = np.random.default_rng(77)


def bits(x):
    return oracle.f32_to_bf16(np.asarray(x, dtype=np.float32))


def val(b):
    return oracle.bf16_to_f32(b).astype(np.float64)


def test_direct_bf16_rounding():
    cases = [
        (1.0 + 2.0 ** -8, 1.0),                        # tie -> even (1.0)
        (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),        # tie -> even
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),   # above the tie: fp32 first would give 1.0
        (-(1.0 + 2.0 ** -8 + 2.0 ** -30), -(1.0 + 2.0 ** -7)),
        (0.0, 0.0),
        (3.0 * 2.0 ** -100, 3.0 * 2.0 ** -100),
        (255.5, 256.0),                                # 255.5 ties between 255 and 256: even = 256
    ]
    for v, want in cases:
        assert val(glue._f64_to_bf16_bits(np.array([v])))[0] == want, v


def test_residual_add_matches_torch_bf16_addition():
    h = bits(RNG.standard_normal((7, 300)) * 3)
    d = bits(RNG.standard_normal((7, 300)))
    th = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16)
    td = torch.from_numpy(d.view(np.int16)).view(torch.bfloat16)
    want = (th + td).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(glue.residual_add(h, d), want)
    np.testing.assert_array_equal(glue.residual_add(h, None), h)


def test_rmsnorm_closed_forms():
    D = 64
    for c in (1.0, -3.0, 0.375, 100.0):
        h = bits(np.full((1, D), c))
        n = val(glue.rmsnorm(h, bits(np.ones(D)), 0.0))
        assert np.all(n == np.sign(c))
        n2 = val(glue.rmsnorm(h, bits(np.full(D, 2.0)), 0.0))
        assert np.all(n2 == 2 * np.sign(c))
    # eps: a constant row c gives h*r = c / sqrt(c^2 + eps)
    h = bits(np.full((1, D), 0.5))
    n = val(glue.rmsnorm(h, bits(np.ones(D)), 0.25))
    assert np.all(n == val(glue._f64_to_bf16_bits(np.array([0.5 / np.sqrt(0.5)]))))


def test_rmsnorm_scale_invariance_and_unit_rms():
    h = bits(RNG.standard_normal((5, 4096)) * 2)
    g = bits(np.ones(4096))
    n = glue.rmsnorm(h, g, 0.0)
    n8 = glue.rmsnorm(bits(val(h) * 8.0), g, 0.0)
    np.testing.assert_array_equal(n, n8)
    rms = np.sqrt(np.mean(val(n) ** 2, axis=1))
    assert np.all(np.abs(rms - 1.0) < 2.0 ** -7)
    # gamma multiplies after the first rounding, per channel
    gv = RNG.uniform(0.5, 2.0, 4096)
    ng = glue.rmsnorm(h, bits(gv), 0.0)
    np.testing.assert_array_equal(ng, glue._f64_to_bf16_bits(val(n) * val(bits(gv))[None, :]))


def test_silu_mul_against_scipy_logistic():
    g = bits(RNG.standard_normal((6, 2000)) * 4)
    u = bits(RNG.standard_normal((6, 2000)))
    a = val(glue.silu_mul(g, u))
    s = val(glue._f64_to_bf16_bits(val(g) * expit(val(g))))
    want = val(glue._f64_to_bf16_bits(s * val(u)))
    # the two silu formulas differ only in the last float64 bits, which can
    # move a bf16 rounding where the value sits on a boundary
    same = a == want
    assert same.mean() > 0.999
    assert np.all(np.abs(a - want) <= 2.0 ** -6 * np.abs(want) + 1e-30)


def test_silu_limits():
    g = bits(np.array([[0.0, 50.0, -50.0, 1.0]]))
    u = bits(np.array([[3.0, 1.0, 1.0, 1.0]]))
    a = val(glue.silu_mul(g, u))[0]
    assert a[0] == 0.0
    assert a[1] == 50.0                       # silu(g) = g for large g
    assert a[2] == val(glue._f64_to_bf16_bits(np.array([-50.0 * np.exp(-50.0)])))[0]
    assert a[3] == val(glue._f64_to_bf16_bits(np.array([1.0 / (1.0 + np.exp(-1.0))])))[0]
