"""Pins of the oracle's stochastic verification (oracle/sample.py) against
what mathematics fixes: the accuracy of its fp32 exp against float64 exp,
closed forms of the acceptance probability and of the inverse-CDF boundaries,
the reduction to greedy verification as T -> 0, and the lossless property of
speculative sampling (the first emitted token follows the verifier's own
softmax, whatever the draft), checked by chi-square tests."""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import sample as S

RNG = np.random.default_rng(20260302)


def softmax64(y, t):
    z = np.asarray(y, dtype=np.float64) / t
    z -= z.max()
    e = np.exp(z)
    return e / e.sum()


# --------------------------------------------------------------------------
# exp_f32
# --------------------------------------------------------------------------

def test_exp_f32_accuracy_against_float64():
    x = np.concatenate([np.linspace(-32, 0, 1_000_001, dtype=np.float32),
                        RNG.uniform(-32, 0, 200_000).astype(np.float32),
                        (-np.arange(47, dtype=np.float32) * np.float32(math.log(2))),
                        np.array([0.0, -0.0, -1e-30, -1e-7, -32.0], dtype=np.float32)])
    x = np.clip(x, -32, 0).astype(np.float32)
    e = S.exp_f32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(e - ref) / ulp) <= 2.0


def test_exp_f32_special_values():
    assert S.exp_f32(np.float32(0.0)) == np.float32(1.0)
    assert S.exp_f32(np.float32(-0.0)) == np.float32(1.0)
    # e^(-k ln 2) is 2^-k, up to the rounding of -k ln 2 to fp32 and 2 ulp
    for k in range(0, 46):
        x = np.float32(-k * math.log(2))
        v = float(S.exp_f32(x))
        rel = abs(float(x) + k * math.log(2)) + 2 * 2.0 ** -23
        assert abs(v - 2.0 ** -k) <= 2.0 ** -k * rel
    with pytest.raises(ValueError):
        S.exp_f32(np.float32(0.5))
    with pytest.raises(ValueError):
        S.exp_f32(np.float32(-33.0))


# --------------------------------------------------------------------------
# fixed-point weights
# --------------------------------------------------------------------------

def test_fixed_weights_track_softmax_numerators():
    y = (RNG.standard_normal(5000) * 3).astype(np.float32)
    for t in (0.25, 0.7, 1.0, 2.0):
        w = S.fixed_weights(y, S.inv_temperature(t))
        assert w.dtype == np.uint64
        assert int(w.max()) == 1 << 40
        assert int(w[np.argmax(y)]) == 1 << 40
        ref = np.exp((y.astype(np.float64) - y.max()) / t) * 2.0 ** 40
        x = (y.astype(np.float64) - y.max()) / t
        # fp32 rounding of (y - m) and of the product with 1/T, the exp's 2 ulp,
        # then the floor
        tol = ref * (np.abs(x) * 4 * 2.0 ** -24 + 3 * 2.0 ** -24) + 1.0
        keep = x > -27
        assert np.all(np.abs(w[keep].astype(np.float64) - ref[keep]) <= tol[keep])
        assert np.all(w[x < -32] == 0)


def test_fixed_weights_uniform_row_and_temperature_scaling():
    y = np.full(100, 3.25, dtype=np.float32)
    w = S.fixed_weights(y, S.inv_temperature(0.9))
    assert np.all(w == 1 << 40)
    # y/T with T a power of two is the same row at T=1 with logits y/T
    y = (RNG.standard_normal(300)).astype(np.float32)
    a = S.fixed_weights(y, S.inv_temperature(0.5))
    b = S.fixed_weights((y * np.float32(2)).astype(np.float32), S.inv_temperature(1.0))
    np.testing.assert_array_equal(a, b)


def test_inv_temperature_validation():
    for bad in (0.0, -1.0, float("inf"), float("nan"), 1e-45):
        with pytest.raises((ValueError, FloatingPointError)):
            S.inv_temperature(bad)


# --------------------------------------------------------------------------
# acceptance and sampling boundaries (closed forms)
# --------------------------------------------------------------------------

def one_seq(y_rows, d, t, ua, us):
    al, nt = S.verify_sample(np.asarray(y_rows, dtype=np.float32), np.array([d]), t,
                             np.array([ua], dtype=np.uint64), np.array([us], dtype=np.uint64))
    return int(al[0]), int(nt[0])


def test_acceptance_boundary_is_the_closed_form():
    V = 50
    for trial in range(20):
        y = (RNG.standard_normal((2, V)) * 2).astype(np.float32)
        t = float(RNG.uniform(0.3, 1.5))
        d = int(RNG.integers(0, V))
        w = S.fixed_weights(y[0], S.inv_temperature(t))
        z = int(w.sum(dtype=np.uint64))
        thr = S.accept_threshold(int(w[d]), z)
        assert 0 < thr <= 1 << 32
        # the probability ceil(W_d 2^32 / Z) / 2^32 is the softmax probability
        p = softmax64(y[0], np.float32(t))[d]
        assert abs(thr / 2.0 ** 32 - p) <= 2.0 ** -32 + 1e-5 * p + 2.0 ** -40 * V
        assert one_seq(y, [d], t, [thr - 1], 0)[0] == 1
        if thr < 1 << 32:
            assert one_seq(y, [d], t, [thr], 0)[0] == 0


def test_sampling_boundaries_are_the_prefix_sums():
    V = 40
    y = (RNG.standard_normal((1, V)) * 1.5).astype(np.float32)
    w = S.fixed_weights(y[0], S.inv_temperature(0.8))
    s = np.cumsum(w, dtype=np.uint64).astype(object)
    z = int(s[-1])
    for j in range(V):
        lo = 0 if j == 0 else int(s[j - 1])
        # smallest u with floor(u z / 2^64) >= lo
        u = -(-(lo << 64) // z)
        assert S.sample_index(w, u) == j or int(w[j]) == 0
        if u > 0:
            assert S.sample_index(w, u - 1) < j or lo == 0
    assert S.sample_index(w, (1 << 64) - 1) == V - 1 - int(np.argmax(w[::-1] > 0))


def test_rejection_removes_the_draft_from_the_residual():
    # two tokens: after rejecting token 0 the next token must be 1
    y = np.array([[2.0, 0.0], [0.0, 0.0]], dtype=np.float32)
    for us in (0, 1 << 63, (1 << 64) - 1):
        al, nt = one_seq(y, [0], 1.0, [(1 << 32) - 1], us)
        assert al == 0 and nt == 1


def test_all_accepted_samples_the_bonus_row():
    V = 6
    y = np.zeros((3, V), dtype=np.float32)
    y[2, 4] = 50.0          # the bonus row is (numerically) a point mass on 4
    al, nt = one_seq(y, [1, 2], 1.0, [0, 0], 12345)
    assert (al, nt) == (2, 4)


def test_out_of_range_draft_is_never_accepted_and_removes_nothing():
    V = 5
    y = np.zeros((2, V), dtype=np.float32)
    y[0, 3] = 60.0
    for d in (-1, V, 1 << 20):
        al, nt = one_seq(y, [d], 1.0, [0], 0)
        assert (al, nt) == (0, 3)


def test_small_temperature_reduces_to_greedy():
    B, G, V = 40, 4, 300
    # logits with distinct values at least 0.05 apart near the top
    y = np.stack([RNG.permutation(V).astype(np.float32) * np.float32(0.05)
                  for _ in range(B * (G + 1))])
    am = oracle.argmax_rows(y).reshape(B, G + 1)
    d = RNG.integers(0, V, size=(B, G)).astype(np.int32)
    for b in range(B):
        p = b % (G + 1)
        d[b, :p] = am[b, :p]
    al_g, nt_g = oracle.greedy_accept(d, am.reshape(-1))
    ua = RNG.integers(0, 1 << 32, size=(B, G), dtype=np.uint64)
    us = RNG.integers(0, 1 << 63, size=B, dtype=np.uint64) * 2 + 1
    al, nt = S.verify_sample(y, d, 1e-3, ua, us)
    np.testing.assert_array_equal(al, al_g)
    np.testing.assert_array_equal(nt, nt_g)


# --------------------------------------------------------------------------
# the lossless property, statistically
# --------------------------------------------------------------------------

def chi2_pvalue(counts, p):
    n = counts.sum()
    exp = p * n
    keep = exp > 0
    assert np.all(counts[~keep] == 0)
    return stats.chisquare(counts[keep], exp[keep]).pvalue


@pytest.mark.parametrize("draft_is_argmax", [False, True])
def test_first_emitted_token_follows_the_verifier(draft_is_argmax):
    V, G, T, N = 7, 1, 0.8, 30000
    y = np.array([[1.0, 0.2, -0.5, 1.3, 0.0, -1.0, 0.7],
                  [0.0, 0.5, 1.0, 0.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    d = 3 if draft_is_argmax else 1
    p = softmax64(y[0], np.float32(T))
    ua = RNG.integers(0, 1 << 32, size=N, dtype=np.uint64)
    us = RNG.integers(0, 1 << 64, size=N, dtype=np.uint64)
    counts = np.zeros(V)
    y_all = np.tile(y, (N, 1))
    al, nt = S.verify_sample(y_all, np.full((N, G), d), T, ua.reshape(N, G), us)
    first = np.where(al >= 1, d, nt)
    np.add.at(counts, first, 1)
    assert chi2_pvalue(counts, p) > 1e-4
    # acceptance rate is p(d)
    assert abs(al.mean() - p[d]) < 5 * math.sqrt(p[d] * (1 - p[d]) / N)


def test_second_token_follows_its_own_row_after_an_accept():
    V, G, T, N = 5, 2, 1.0, 30000
    y = np.array([[2.0, 0.0, 0.0, 0.0, 0.0],     # row 0: draft 0 accepted often
                  [0.0, 1.0, 0.5, -0.5, 0.2],     # row 1: after position 0
                  [0.0, 0.0, 0.0, 0.0, 3.0]], dtype=np.float32)
    d = np.array([[0, 2]] * N)
    ua = RNG.integers(0, 1 << 32, size=(N, G), dtype=np.uint64)
    us = RNG.integers(0, 1 << 64, size=N, dtype=np.uint64)
    al, nt = S.verify_sample(np.tile(y, (N, 1)), d, T, ua, us)
    # among sequences that accepted d0, the second emitted token is d1 if
    # accepted, else the sampled token: its law must be row 1's softmax
    sel = al >= 1
    second = np.where(al[sel] >= 2, 2, nt[sel])
    counts = np.bincount(second, minlength=V).astype(float)
    assert chi2_pvalue(counts, softmax64(y[1], T)) > 1e-4
    # and the bonus token after two accepts follows row 2
    bonus = nt[al == 2]
    assert len(bonus) > 1000
    counts = np.bincount(bonus, minlength=V).astype(float)
    assert chi2_pvalue(counts, softmax64(y[2], T)) > 1e-4
