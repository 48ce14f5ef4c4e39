"""GPU parity of the W4A8 path (int4 per-channel weights, through the C
ABI) against the oracle (oracle.quantize_weight_int4 + the exact integer
contraction and dequant) on the same seeded inputs.

Bars: int4 codes (read back through the documented int4 tiled layout),
scales, int32 accumulators, fp32 dequant and bf16 outputs bit-exact; bf16
also within 1e-2 relative / 1e-3 absolute of the oracle's fp32; argmax,
accepted lengths and next tokens exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import announce, dev, dev_bf16, gpu_available, host

pytestmark = pytest.mark.gpu

if gpu_available():
    import w8a8_quantized_verification_amd as w8

W_W4 = 7   # seed space of these tests


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no ROCm GPU")


def untile_w4(t: np.ndarray, N: int, K: int, full: bool = False) -> np.ndarray:
    """Codes int8 [N][K] from the int4 tiled buffer [tiles][pairs][64][16]
    (layout of include/w8a8.h: lane l = channel l%16 + 16 * k-group; bytes
    0..7 for the first 64 k of the pair, 8..15 for the second; in each half,
    word wi byte i holds j = 4*wi + i (low nibble) and j = 8 + 4*wi + i
    (high nibble))."""
    tiles, pairs = t.shape[0], t.shape[1]
    u = t.view(np.uint8).reshape(tiles, pairs, 4, 16, 2, 2, 4)   # tile pair g col half wi i
    lo = (u & 0xF).astype(np.int16)
    hi = (u >> 4).astype(np.int16)
    lo = ((lo ^ 8) - 8).astype(np.int8)
    hi = ((hi ^ 8) - 8).astype(np.int8)
    j16 = np.empty((tiles, pairs, 4, 16, 2, 16), dtype=np.int8)
    j16[..., 0:8] = lo.reshape(tiles, pairs, 4, 16, 2, 8)       # j = 4*wi + i
    j16[..., 8:16] = hi.reshape(tiles, pairs, 4, 16, 2, 8)      # j = 8 + 4*wi + i
    a = j16.transpose(0, 3, 1, 4, 2, 5)                          # tile col pair half g j
    a = a.reshape(tiles * 16, pairs * 128)
    return a if full else a[:N, :K]


@pytest.mark.parametrize("N,K,smooth", [(512, 256, False), (1000, 4096, False), (17, 25600, False),
                                        (33, 80, False), (5, 16, False), (300, 12288, True),
                                        (64, 1040, True), (3, 0, False)])
def test_quantize_weight_w4(N, K, smooth):
    announce(f"quantize_weight_w4 N={N} K={K} smooth={smooth}")
    w = synth.weights_f32(W_W4, N, K)
    if K > 0:
        w[0, :] = 0.0                      # an all-zero channel
        w[1 % N, 5 % K] = 3.0              # an outlier
    s = synth.smoothing_vector(W_W4, K) if smooth and K > 0 else None
    q_ref, s_ref = oracle.quantize_weight_int4(w, smooth=s)
    wq4, ws = w8.quantize_weight_w4(dev(w), None if s is None else dev(s))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ws).view(np.uint32), s_ref.view(np.uint32))
    if K == 0:
        return
    t = host(wq4)
    full = untile_w4(t, N, K, full=True)
    np.testing.assert_array_equal(full[:N, :K], q_ref)
    assert not full[N:].any() and not full[:, K:].any()          # padding is zero
    assert t.nbytes == (N + 15) // 16 * 16 * ((K + 127) // 128) * 64


def run_w4_case(M, N, K, seed):
    bits = synth.activations_bf16(seed, M, K, outliers=K > 0)
    w = synth.weights_f32(seed, N, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    q_r, s_r = oracle.quantize_weight_int4(w)
    acc_r, y32_r, y_r = oracle.w8a8_linear(xq_r, xs_r, q_r, s_r)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wq4, ws = w8.quantize_weight_w4(dev(w))
    yb, yf, acc = w8.linear_w4(xq, xs, wq4, ws, want_bf16=True, want_f32=True, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), acc_r)
    np.testing.assert_array_equal(host(yf).view(np.uint32), y32_r.view(np.uint32))
    np.testing.assert_array_equal(host(yb), y_r)
    y = oracle.bf16_to_f32(host(yb)).astype(np.float64)
    assert np.all(np.abs(y - y32_r) <= 1e-3 + 1e-2 * np.abs(y32_r.astype(np.float64)))


W4_CASES = [
    (5, 512, 256), (5, 4096, 4096), (5, 1024, 4096), (5, 12288, 4096), (5, 4096, 12288),
    (8, 8192, 5120), (8, 5120, 25600), (1, 1000, 4096), (16, 777, 1040), (3, 17, 16),
    (5, 1, 4096), (17, 300, 512), (40, 257, 2048), (5, 64, 0), (5, 48, 80),
]


@pytest.mark.parametrize("M,N,K", W4_CASES)
def test_linear_w4(M, N, K):
    announce(f"linear_w4 M={M} N={N} K={K}")
    run_w4_case(M, N, K, seed=300 + M + N % 97 + K % 89)


def test_linear_w4_extreme_accumulators():
    """Every code at the int4 limit with every activation at +-127 and the
    largest K: |acc| = 127 * 7 * K (the kernel accumulates 16x that)."""
    M, N, K = 3, 20, 133136
    announce(f"linear_w4 extremes K={K}")
    w = np.ones((N, K), dtype=np.float32)
    w[1::2] *= -1.0
    bits = oracle.f32_to_bf16(np.where(np.arange(M)[:, None] % 2 == 0, 1.0, -1.0)
                              * np.ones((M, K), dtype=np.float32))
    xq_r, xs_r = oracle.quantize_act(bits)
    q_r, s_r = oracle.quantize_weight_int4(w)
    acc_r, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, q_r, s_r)
    assert abs(int(acc_r[0, 0])) == 127 * 7 * K
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wq4, ws = w8.quantize_weight_w4(dev(w))
    _, yf, acc = w8.linear_w4(xq, xs, wq4, ws, want_bf16=False, want_f32=True, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), acc_r)
    np.testing.assert_array_equal(host(yf).view(np.uint32), y32_r.view(np.uint32))


@pytest.mark.parametrize("B,G,V,K", [(1, 4, 512, 256), (1, 4, 151936, 4096), (3, 7, 5000, 5120),
                                     (2, 3, 17, 64), (32, 8, 4099, 1024)])
def test_lm_head_argmax_w4(B, G, V, K):
    announce(f"lm_head_argmax_w4 B={B} G={G} V={V} K={K}")
    R = B * (G + 1)
    bits = synth.activations_bf16(W_W4, R, K)
    w = synth.weights_f32(W_W4 + 1, V, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    q_r, s_r = oracle.quantize_weight_int4(w)
    _, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, q_r, s_r)
    am_r = oracle.argmax_rows(y32_r).reshape(B, G + 1)
    draft = synth.draft_ids(W_W4, B, G, V)
    for b in range(B):
        p = b % (G + 1)
        draft[b, :p] = am_r[b, :p]
    am_r, al_r, nt_r = oracle.verify_accept(y32_r, draft)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wq4, ws = w8.quantize_weight_w4(dev(w))
    wsp = w8.Workspace()
    lg = w8.lm_head_argmax_w4(xq, xs, wq4, ws, logits=torch.empty(R, V, dtype=torch.float32,
                                                                  device="cuda:0"), workspace=wsp)
    am, al, nt = w8.accept_from_keys(dev(draft), workspace=wsp)
    w8.lm_head_argmax_w4(xq, xs, wq4, ws, workspace=wsp)          # again, no logits
    am2, al2, nt2 = w8.accept_from_keys(dev(draft), workspace=wsp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(lg).view(np.uint32), y32_r.view(np.uint32))
    for a, l, n in ((am, al, nt), (am2, al2, nt2)):
        np.testing.assert_array_equal(host(a), am_r)
        np.testing.assert_array_equal(host(l), al_r)
        np.testing.assert_array_equal(host(n), nt_r)
