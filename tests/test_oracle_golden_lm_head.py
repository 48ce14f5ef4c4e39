"""Checks of the stored LM-head verdicts (tests/golden/lm_head_m5_1000.txt)
on the CPU: internal consistency of every trial, and two trials recomputed
end to end with the oracle at full size (K = 4096, V = 151936)."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.test_gpu_lm_head_1000 import K, M, V, load_golden

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lm_head_m5_1000.txt")


def test_golden_trials_are_consistent():
    meta, rows = load_golden()
    assert len(rows) == 1000 and [r["t"] for r in rows] == list(range(1000))
    known = 0
    for r in rows:
        p, d, a_ref, am = r["p"], r["draft"], r["a_ref"], r["am"]
        assert p == r["t"] % M
        assert np.array_equal(d[:p], a_ref[:p])          # the built-in prefix
        if p < M - 1:
            assert d[p] != a_ref[p]                       # and the built-in mismatch
        al, nt = oracle.greedy_accept(d[None, :], am)
        assert (al[0], nt[0]) == (r["accept_len"], r["next_token"])
        if np.array_equal(am[:p + 1], a_ref[:p + 1]):
            known += 1
            assert r["accept_len"] == p                   # the accepted-length identity
        # the drafts regenerate from their seed
        d2 = synth.prefix_drafts(a_ref, p, V, synth.rng(synth.W_LM_HEAD, synth.T_DRAFT, r["t"]))
        assert np.array_equal(d2, d)
    assert known >= 800


def test_two_trials_recomputed_by_the_oracle():
    meta, rows = load_golden()
    picks = [7, 993]
    w = synth.weights_f32(synth.W_LM_HEAD, V, K)
    wq, ws = oracle.quantize_weight(w)
    del w
    import hashlib
    assert hashlib.sha256(ws.tobytes()).hexdigest() == meta["w_scale_sha256"]
    x = np.concatenate([synth.activations_bf16(synth.W_LM_HEAD, M, K, index=t) for t in picks])
    xq, xs = oracle.quantize_act(x)
    _, y32, _ = oracle.w8a8_linear(xq, xs, wq, ws)
    am = oracle.argmax_rows(y32).reshape(len(picks), M)
    for i, t in enumerate(picks):
        assert np.array_equal(am[i], rows[t]["am"])
