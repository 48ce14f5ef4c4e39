"""GPU parity of stochastic verification (w8a8_verify_sample, through the C
ABI) and of its fixed-point softmax weights (w8a8_sample_weights) against
the oracle (oracle/sample.py) on the same seeded inputs.

Bars: every weight W_j bit-exact; accept_len and next_token exact, including
random words placed exactly on the acceptance and inverse-CDF boundaries the
oracle computes."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import sample as S
from tests.gpu_util import announce, dev, gpu_available, host

pytestmark = pytest.mark.gpu

if gpu_available():
    import w8a8_quantized_verification_amd as w8

W_SAMPLE = 6      # seed space of these tests


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no ROCm GPU")


def logits_rows(R, V, index, scale=1.3):
    return (synth.rng(W_SAMPLE, 10, index).standard_normal((R, V), dtype=np.float32)
            * np.float32(scale)).astype(np.float32)


def words(index, shape, bits):
    r = synth.rng(W_SAMPLE, 11, index)
    if bits == 32:
        return r.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32)
    return r.integers(0, 1 << 64, size=shape, dtype=np.uint64)


def gpu_sample(y, d, t, ua, us):
    B, G = d.shape
    ua_t = torch.from_numpy(ua.astype(np.uint32).view(np.int32).reshape(B, G).copy()).cuda()
    us_t = torch.from_numpy(np.asarray(us, dtype=np.uint64).view(np.int64).copy()).cuda()
    al, nt = w8.verify_sample(dev(y), dev(d.astype(np.int32)), t, ua_t, us_t)
    torch.cuda.synchronize()
    return host(al), host(nt)


@pytest.mark.parametrize("R,V,t", [(7, 5000, 1.0), (3, 151936, 0.7), (4, 2049, 1.7),
                                   (2, 1, 1.0), (5, 4096, 0.05), (1, 300, 25.0)])
def test_sample_weights_bit_exact(R, V, t):
    announce(f"sample_weights R={R} V={V} T={t}")
    y = logits_rows(R, V, R * 1000 + V)
    if V > 10:
        y[0, :5] = y[0].max()            # ties at the maximum
        y[-1, 7] = -1e4                  # far below: weight 0
        y[-1, 8] = np.float32(-0.0)
        y[-1, 9] = np.float32(0.0)
    w = host(w8.sample_weights(dev(y), t)).view(np.uint64)
    inv_t = S.inv_temperature(t)
    for r in range(R):
        np.testing.assert_array_equal(w[r], S.fixed_weights(y[r], inv_t))


def test_sample_weights_exp_grid():
    """Every fp32 exponent argument on a dense grid of [-32, 0]: one row per
    slice, max 0 in every row, so x_j = y_j at T = 1."""
    x = np.linspace(-32, 0, 1 << 20, dtype=np.float32).reshape(16, -1).copy()
    x[:, -1] = 0.0
    w = host(w8.sample_weights(dev(x), 1.0)).view(np.uint64)
    ref = np.stack([S.fixed_weights(x[r], np.float32(1.0)) for r in range(16)])
    np.testing.assert_array_equal(w, ref)


@pytest.mark.parametrize("B,G,V,t", [(32, 8, 4099, 1.0), (32, 8, 4099, 0.3), (1, 4, 151936, 1.0),
                                     (3, 7, 151936, 0.7), (4, 0, 1000, 1.0), (5, 15, 2048, 1.3),
                                     (2, 3, 1, 1.0)])
def test_verify_sample_random(B, G, V, t):
    announce(f"verify_sample B={B} G={G} V={V} T={t}")
    y = logits_rows(B * (G + 1), V, B * 7 + G * 13 + V, scale=2.0)
    am = oracle.argmax_rows(y).reshape(B, G + 1)
    d = synth.rng(W_SAMPLE, 12, V).integers(0, V, size=(B, G)).astype(np.int32)
    for b in range(B):                    # spread the accepted lengths
        p = b % (G + 1)
        d[b, :p] = am[b, :p]
    ua = words(B + G, (B, G), 32)
    us = words(B + G + 1, (B,), 64)
    al_r, nt_r = S.verify_sample(y, d, t, ua, us)
    al, nt = gpu_sample(y, d, t, ua, us)
    np.testing.assert_array_equal(al, al_r)
    np.testing.assert_array_equal(nt, nt_r)


def test_verify_sample_exact_boundaries():
    """Random words placed on the oracle's acceptance threshold and on every
    inverse-CDF boundary of a small vocabulary."""
    announce("verify_sample boundaries")
    V, G = 37, 1
    y = logits_rows(2, V, 99, scale=1.5)
    t = 0.9
    inv_t = S.inv_temperature(t)
    w0 = S.fixed_weights(y[0], inv_t)
    z0 = int(w0.sum(dtype=np.uint64))
    cases_d, cases_ua, cases_us = [], [], []
    for d in (0, 5, int(np.argmax(y[0])), 36):
        thr = S.accept_threshold(int(w0[d]), z0)
        for ua in (thr - 1, thr, 0, (1 << 32) - 1):
            if 0 <= ua < 1 << 32:
                # after a rejection at d: every boundary of the residual
                res = w0.copy()
                res[d] = 0
                s = np.cumsum(res, dtype=np.uint64)
                zr = int(s[-1])
                for j in range(0, V, 3):
                    lo = 0 if j == 0 else int(s[j - 1])
                    u = -(-(lo << 64) // zr)
                    for us in (u - 1, u):
                        if 0 <= us < 1 << 64:
                            cases_d.append(d)
                            cases_ua.append(ua)
                            cases_us.append(us)
    n = len(cases_d)
    yy = np.tile(y, (n, 1))
    d = np.array(cases_d, dtype=np.int32).reshape(n, G)
    ua = np.array(cases_ua, dtype=np.uint64).reshape(n, G)
    us = np.array(cases_us, dtype=np.uint64)
    al_r, nt_r = S.verify_sample(yy, d, t, ua, us)
    al, nt = gpu_sample(yy, d, t, ua, us)
    np.testing.assert_array_equal(al, al_r)
    np.testing.assert_array_equal(nt, nt_r)
    assert 0 < al_r.sum() < n                 # both outcomes exercised


def test_verify_sample_edge_cases():
    announce("verify_sample edge cases")
    V, G = 50, 3
    y = logits_rows(4 * (G + 1), V, 5)
    y[0:G + 1, 10] = 80.0                       # sequence 0: all mass on token 10
    d = np.array([[10, 10, 10],                 # always accepted -> bonus ~ row 3 = token 10
                  [-5, 3, 4],                   # out of range: never accepted
                  [V, 1, 2],                    # out of range (= V)
                  [0, 1, 2]], dtype=np.int32)
    ua = np.array([[(1 << 32) - 1] * 3, [0] * 3, [0] * 3, [0] * 3], dtype=np.uint64)
    us = np.array([0, (1 << 64) - 1, 1 << 63, 12345], dtype=np.uint64)
    al_r, nt_r = S.verify_sample(y, d, 1.0, ua, us)
    al, nt = gpu_sample(y, d, 1.0, ua, us)
    assert (al_r[0], nt_r[0]) == (3, 10)
    assert al_r[1] == 0 and al_r[2] == 0
    np.testing.assert_array_equal(al, al_r)
    np.testing.assert_array_equal(nt, nt_r)


def test_verify_sample_small_temperature_matches_greedy():
    announce("verify_sample T -> 0 equals verify_accept")
    B, G, V = 16, 4, 3000
    perm = [synth.rng(W_SAMPLE, 13, i).permutation(V) for i in range(B * (G + 1))]
    y = (np.stack(perm).astype(np.float32) * np.float32(0.05)).astype(np.float32)
    am = oracle.argmax_rows(y).reshape(B, G + 1)
    d = synth.rng(W_SAMPLE, 14, 0).integers(0, V, size=(B, G)).astype(np.int32)
    for b in range(B):
        d[b, :b % (G + 1)] = am[b, :b % (G + 1)]
    _, al_g, nt_g = w8.verify_accept(dev(y), dev(d))
    al, nt = gpu_sample(y, d, 1e-3, words(7, (B, G), 32), words(8, (B,), 64))
    np.testing.assert_array_equal(al, host(al_g))
    np.testing.assert_array_equal(nt, host(nt_g))


def test_verify_sample_after_w8a8_lm_head():
    """The full stochastic step on the W8A8 path: quantize_act -> LM-head
    linear (fp32 logits) -> verify_sample, against the oracle's own chain."""
    announce("quantize_act -> linear -> verify_sample, V=8192 K=1024")
    B, G, V, K, t = 4, 4, 8192, 1024, 1.0
    bits = synth.activations_bf16(W_SAMPLE, B * (G + 1), K)
    w = synth.weights_f32(W_SAMPLE, V, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    wq_r, ws_r = oracle.quantize_weight(w)
    _, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    am = oracle.argmax_rows(y32_r).reshape(B, G + 1)
    d = synth.draft_ids(W_SAMPLE, B, G, V)
    for b in range(B):
        d[b, :b + 1] = am[b, :b + 1]
    ua, us = words(20, (B, G), 32), words(21, (B,), 64)
    al_r, nt_r = S.verify_sample(y32_r, d, t, ua, us)
    from tests.gpu_util import dev_bf16
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wt, wsc = w8.quantize_weight(dev(w), tiled=True)
    _, yf, _ = w8.linear(xq, xs, wt, wsc, want_bf16=False, want_f32=True)
    torch.cuda.synchronize()
    al, nt = gpu_sample(host(yf), d, t, ua, us)
    np.testing.assert_array_equal(al, al_r)
    np.testing.assert_array_equal(nt, nt_r)
