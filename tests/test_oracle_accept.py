"""Pins for the oracle's argmax and greedy acceptance.

* argmax: brute-force loop, constructed ties (lowest index wins, also across
  a 1024-wide chunk boundary), -0 == +0, non-finite rejected;
* acceptance: exhaustive over all 2^G match patterns for G = 4 and G = 8
  against a hand-written rule (accept_len = index of the first mismatch);
* the identity: where the W8A8 argmax equals the bf16-reference argmax on
  positions 0..p, drafts built from the reference's first p ids are accepted
  to length exactly p (small LM head, many trials).
"""
import itertools

import numpy as np
import pytest

import synth
from oracle import (argmax_rows, bf16_reference_logits, greedy_accept, quantize_act,
                    quantize_weight, verify_accept, w8a8_linear)


def brute_argmax(row):
    best, idx = row[0], 0
    for i in range(1, len(row)):
        if row[i] > best:
            best, idx = row[i], i
    return idx


def test_argmax_brute_force():
    r = np.random.default_rng(1)
    y = r.standard_normal((40, 777)).astype(np.float32)
    # quantize values so that ties happen often
    y = np.round(y * 4).astype(np.float32)
    got = argmax_rows(y)
    assert got.dtype == np.int32
    for i in range(y.shape[0]):
        assert got[i] == brute_argmax(list(y[i]))


def test_argmax_constructed_ties():
    y = np.zeros((4, 3000), dtype=np.float32)
    y[0, [3, 7]] = 5.0                 # tie -> 3
    y[1, [2047, 1023, 1024]] = 2.0     # tie across a 1024-wide chunk boundary -> 1023
    y[2, :] = -1.0                     # all equal -> 0
    y[3, 2999] = 1e-30                 # last element alone
    np.testing.assert_array_equal(argmax_rows(y), [3, 1023, 0, 2999])


def test_argmax_signed_zero_and_negative_rows():
    y = np.array([[-0.0, 0.0, -1.0], [-3.0, -2.0, -2.0], [0.0, -0.0, -0.0]], dtype=np.float32)
    np.testing.assert_array_equal(argmax_rows(y), [0, 1, 0])


def test_argmax_rejects_non_finite():
    with pytest.raises(ValueError):
        argmax_rows(np.array([[1.0, np.nan]], dtype=np.float32))


def rule_accept(d, a):
    """accept_len = index of the first position whose draft differs from the
    target's argmax (G if none); next = target argmax there."""
    G = len(d)
    mism = [i for i in range(G) if d[i] != a[i]]
    n = mism[0] if mism else G
    return n, a[n]


@pytest.mark.parametrize("G", [1, 4, 8])
def test_accept_exhaustive_patterns(G):
    r = np.random.default_rng(G)
    pats = list(itertools.product([0, 1], repeat=G))
    B = len(pats)
    a = r.integers(0, 1000, size=(B, G + 1)).astype(np.int32)
    d = np.empty((B, G), dtype=np.int32)
    for b, pat in enumerate(pats):
        for i, match in enumerate(pat):
            d[b, i] = a[b, i] if match else (a[b, i] + 1 + r.integers(0, 5)) % 1000
    al, nt = greedy_accept(d, a.reshape(-1))
    for b in range(B):
        n, nx = rule_accept(list(d[b]), list(a[b]))
        assert al[b] == n and nt[b] == nx
    # all-match rows accept G and take the bonus token at position G
    full = [b for b, p in enumerate(pats) if all(p)]
    assert al[full[0]] == G and nt[full[0]] == a[full[0], G]


def test_accept_out_of_range_drafts_never_match():
    a = np.array([5, 6, 7], dtype=np.int32)
    al, nt = greedy_accept(np.array([[-1, 6]], np.int32), a)
    assert al[0] == 0 and nt[0] == 5


def test_verify_accept_composes():
    y = np.zeros((5, 10), dtype=np.float32)
    for i, j in enumerate([3, 1, 4, 1, 5]):
        y[i, j] = 1.0
    am, al, nt = verify_accept(y, np.array([[3, 1, 9, 9]], np.int32))
    np.testing.assert_array_equal(am, [3, 1, 4, 1, 5])
    assert al[0] == 2 and nt[0] == 4


def test_accept_length_identity_on_small_lm_head():
    """Drafts match the bf16-reference argmax for the first p positions.
    Whenever the W8A8 argmax agrees with the reference on positions 0..p,
    the accepted length is exactly p; every other trial is counted."""
    K, V, G = 256, 512, 4
    w = synth.weights_f32(77, V, K)
    wq, ws = quantize_weight(w)
    agree_trials = 0
    for t in range(100):
        x = synth.activations_bf16(77, G + 1, K, index=t)
        a_ref = np.argmax(bf16_reference_logits(x, w), axis=1)
        p = t % (G + 1)
        d = synth.prefix_drafts(a_ref, p, V, synth.rng(77, synth.T_DRAFT, t))
        assert np.array_equal(d[:p], a_ref[:p])
        if p < G:
            assert d[p] != a_ref[p]
        xq, xs = quantize_act(x)
        _, y32, _ = w8a8_linear(xq, xs, wq, ws)
        am, al, _ = verify_accept(y32, d[None, :])
        if np.array_equal(am[:p + 1], a_ref[:p + 1]):
            agree_trials += 1
            assert al[0] == p
    assert agree_trials >= 60
