"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on
the same seeded inputs.

Bars: int8 codes, scales, int32 accumulators, fp32 dequant (y32), argmax,
accepted lengths and next tokens are bit-exact (every fp32 step is pinned:
single correctly rounded operations in a fixed order); bf16 outputs are
checked bit-exact too, and also against the oracle's fp32 dequant within
1e-2 relative / 1e-3 absolute, the stated tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import announce, dev, dev_bf16, gpu_available, host

pytestmark = pytest.mark.gpu

if gpu_available():
    import w8a8_quantized_verification_amd as w8


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no ROCm GPU")


def assert_bf16_tolerance(y_bits, y32_oracle):
    y = oracle.bf16_to_f32(y_bits).astype(np.float64)
    ref = y32_oracle.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 1e-3 + 1e-2 * np.abs(ref))


# --------------------------------------------------------------------------
# quantize_act / quantize_weight
# --------------------------------------------------------------------------

ACT_SHAPES = [(5, 256), (5, 4096), (5, 12288), (8, 25600), (288, 4096), (7, 16), (1, 2064),
              (3, 0), (0, 64)]


@pytest.mark.parametrize("M,K", ACT_SHAPES)
@pytest.mark.parametrize("outliers", [False, True])
def test_quantize_act(M, K, outliers):
    announce(f"quantize_act M={M} K={K} outliers={outliers}")
    bits = synth.activations_bf16(101, M, K, outliers=outliers and K > 0)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_act(bits)
    np.testing.assert_array_equal(host(xq), q_ref)
    np.testing.assert_array_equal(host(xs).view(np.uint32), s_ref.view(np.uint32))


def test_quantize_act_degenerate_rows():
    announce("quantize_act degenerate rows")
    K = 256
    x = np.random.default_rng(5).standard_normal((6, K)).astype(np.float32)
    x[0] = 0.0                       # all zero -> scale 0, codes 0
    x[1] = -0.0
    x[2] = 0.0
    x[2, 17] = 1e-38                 # 127/amax overflows: zeros stay 0, nonzeros saturate
    x[2, 18] = -3e-39
    x[3] = 0.0
    x[3, 255] = -5.0                 # single nonzero at the last column
    x[4] = np.float32(2.0 ** -130)   # subnormal row
    x[5, :8] = [254, 1, 5, 3, -5, -3, 127, -127]  # rounding ties with inv = 0.5
    x[5, 8:] = 0
    bits = synth.to_bf16_bits(x)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_act(bits)
    np.testing.assert_array_equal(host(xq), q_ref)
    np.testing.assert_array_equal(host(xs).view(np.uint32), s_ref.view(np.uint32))
    assert list(q_ref[5, :8]) == [127, 0, 2, 2, -2, -2, 64, -64]


@pytest.mark.parametrize("M,K", [(5, 4096), (288, 1024)])
def test_quantize_act_smoothing(M, K):
    announce(f"quantize_act smoothing M={M} K={K}")
    bits = synth.activations_bf16(102, M, K, outliers=True)
    s = synth.smoothing_vector(102, K)
    xq, xs = w8.quantize_act(dev_bf16(bits), dev(s))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_act(bits, smooth=s)
    np.testing.assert_array_equal(host(xq), q_ref)
    np.testing.assert_array_equal(host(xs).view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("N,K", [(512, 256), (1000, 4096), (300, 12288), (17, 25600), (5, 0)])
@pytest.mark.parametrize("smooth", [False, True])
def test_quantize_weight(N, K, smooth):
    announce(f"quantize_weight N={N} K={K} smooth={smooth}")
    w = synth.weights_f32(103, N, K)
    if N > 3 and K > 0:
        w[3] = 0.0
    s = synth.smoothing_vector(103, K) if smooth else None
    wq, ws = w8.quantize_weight(dev(w), None if s is None else dev(s))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_weight(w, smooth=s)
    np.testing.assert_array_equal(host(wq), q_ref)
    np.testing.assert_array_equal(host(ws).view(np.uint32), s_ref.view(np.uint32))


# --------------------------------------------------------------------------
# w8a8_linear
# --------------------------------------------------------------------------

def run_linear_case(M, N, K, seed, outliers=True):
    bits = synth.activations_bf16(seed, M, K, outliers=outliers and K > 0)
    w = synth.weights_f32(seed, N, K)
    xq_ref, xs_ref = oracle.quantize_act(bits)
    wq_ref, ws_ref = oracle.quantize_weight(w)
    acc_ref, y32_ref, y_ref = oracle.w8a8_linear(xq_ref, xs_ref, wq_ref, ws_ref)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wq, ws = w8.quantize_weight(dev(w))
    yb, yf, acc = w8.linear(xq, xs, wq, ws, want_bf16=True, want_f32=True, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), acc_ref)
    np.testing.assert_array_equal(host(yf).view(np.uint32), y32_ref.view(np.uint32))
    np.testing.assert_array_equal(host(yb), y_ref)
    assert_bf16_tolerance(host(yb), y32_ref)
    return xq, xs, wq, ws


LINEAR_CASES = [
    (5, 512, 256),        # the tiny verify linear
    (5, 4096, 4096),      # q / o
    (5, 1024, 4096),      # k / v
    (5, 12288, 4096),     # gate / up
    (5, 4096, 12288),     # down
    (8, 8192, 5120),      # Qwen3-32B q
    (8, 5120, 25600),     # Qwen3-32B down
    (1, 1000, 4096),      # one token, ragged N
    (16, 777, 1040),      # full 16-row tile, ragged N and a partial 64-wide K step
    (3, 17, 16),          # one 16-byte k group
    (5, 1, 4096),         # a single output channel
    (17, 300, 512),       # two row blocks
    (40, 257, 2048),      # three row blocks, ragged
    (5, 64, 0),           # empty contraction
]


@pytest.mark.parametrize("M,N,K", LINEAR_CASES)
def test_linear(M, N, K):
    announce(f"linear M={M} N={N} K={K}")
    run_linear_case(M, N, K, seed=200 + M + N % 97 + K % 89)


def test_linear_outputs_subsets_and_workspace_reuse():
    """Each output alone matches; repeated split-K calls on one workspace stay
    exact (the workspace is left zero-filled after every call)."""
    announce("linear output subsets + split-K workspace reuse")
    M, N, K = 5, 1024, 4096
    xq, xs, wq, ws = run_linear_case(M, N, K, seed=301)
    assert w8.linear_workspace_bytes(M, N, K) > 0
    ref_b, ref_f, ref_a = (host(t) for t in w8.linear(xq, xs, wq, ws, want_bf16=True,
                                                         want_f32=True, want_acc=True))
    for _ in range(5):
        yb, _, _ = w8.linear(xq, xs, wq, ws, want_bf16=True)
        _, yf, _ = w8.linear(xq, xs, wq, ws, want_bf16=False, want_f32=True)
        _, _, acc = w8.linear(xq, xs, wq, ws, want_bf16=False, want_acc=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(yb), ref_b)
        np.testing.assert_array_equal(host(yf), ref_f)
        np.testing.assert_array_equal(host(acc), ref_a)


def test_linear_extreme_accumulators():
    """All-(+127) activations against +-127 weights at K = 25600: the int32
    accumulator reaches +-16129*K = +-412,902,400 exactly."""
    announce("linear extreme accumulators")
    M, N, K = 5, 48, 25600
    xq = torch.full((M, K), 127, dtype=torch.int8, device="cuda:0")
    wq = torch.full((N, K), -127, dtype=torch.int8, device="cuda:0")
    wq[1::2] = 127
    xs = torch.ones(M, dtype=torch.float32, device="cuda:0")
    ws = torch.ones(N, dtype=torch.float32, device="cuda:0")
    _, _, acc = w8.linear(xq, xs, wq, ws, want_bf16=False, want_acc=True)
    torch.cuda.synchronize()
    a = host(acc)
    assert np.all(a[:, 0::2] == -16129 * K) and np.all(a[:, 1::2] == 16129 * K)


def test_linear_batched_m288_sampled():
    """Batched verification, M = 32 x (8+1) = 288 on the q shape: the full
    int32 result against the oracle."""
    announce("linear M=288 q shape")
    run_linear_case(288, 4096, 4096, seed=302)


# --------------------------------------------------------------------------
# verify_accept
# --------------------------------------------------------------------------

def run_verify_case(logits, draft):
    am_ref, al_ref, nt_ref = oracle.verify_accept(logits, draft)
    am, al, nt = w8.verify_accept(dev(logits), dev(draft))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(am), am_ref)
    np.testing.assert_array_equal(host(al), al_ref)
    np.testing.assert_array_equal(host(nt), nt_ref)
    return al_ref


@pytest.mark.parametrize("B,G,V", [(1, 4, 512), (1, 4, 151936), (32, 8, 151936), (1, 7, 151936),
                                   (3, 0, 1000), (2, 3, 1), (4, 2, 4097), (1, 255, 300)])
def test_verify_accept_random(B, G, V):
    announce(f"verify_accept B={B} G={G} V={V}")
    r = np.random.default_rng(B * 1000 + G * 10 + V % 1000)
    logits = r.standard_normal((B * (G + 1), V)).astype(np.float32)
    am = oracle.argmax_rows(logits).reshape(B, G + 1)
    draft = synth.draft_ids(400, B, G, V)
    # make every acceptance length 0..G occur: copy a prefix of the argmax
    for b in range(B):
        p = b % (G + 1)
        draft[b, :p] = am[b, :p]
    run_verify_case(logits, draft)


def test_verify_accept_ties_and_boundaries():
    announce("verify_accept ties")
    V = 3 * 4096 + 5
    logits = np.zeros((5, V), dtype=np.float32)
    logits[0, [4095, 4096, 9000]] = 7.0          # tie across a chunk boundary -> 4095
    logits[1, :] = -2.0                          # all equal -> 0
    logits[2, [V - 1]] = 1e-30                   # the ragged tail holds the max
    logits[3, [0, V - 1]] = 3.0                  # first and last
    logits[4, 8192] = -0.0                       # -0 == +0: lowest index (0) wins
    draft = np.array([[4095, 0, 17, 0]], dtype=np.int32)
    al = run_verify_case(logits, draft)
    assert al[0] == 2


def test_verify_accept_out_of_range_drafts():
    announce("verify_accept out-of-range drafts")
    logits = np.random.default_rng(9).standard_normal((9, 600)).astype(np.float32)
    draft = np.array([[-1, 600, 10**9, 5, 5, 5, 5, 5]], dtype=np.int32)
    run_verify_case(logits, draft)


# --------------------------------------------------------------------------
# bf16 reference linear
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(5, 512, 256), (5, 4096, 4096), (8, 1000, 5120), (16, 33, 48)])
def test_bf16_reference_linear(M, N, K):
    announce(f"bf16 linear M={M} N={N} K={K}")
    bits = synth.activations_bf16(500, M, K, outliers=True)
    w = synth.weights_f32(500, N, K)
    wb = synth.to_bf16_bits(w)
    ref = oracle.bf16_reference_logits(bits, w)
    _, yf = w8.bf16_linear(dev_bf16(bits), dev_bf16(wb), want_bf16=False, want_f32=True)
    torch.cuda.synchronize()
    x64 = np.abs(oracle.bf16_to_f32(bits).astype(np.float64))
    w64 = np.abs(oracle.bf16_to_f32(wb).astype(np.float64))
    bound = K * 2.0 ** -23 * (x64 @ w64.T)
    assert np.all(np.abs(host(yf).astype(np.float64) - ref) <= bound)


# --------------------------------------------------------------------------
# one verify step end to end (tiny workload)
# --------------------------------------------------------------------------

def test_tiny_verify_step_end_to_end():
    """M=5, K=256, N=V=512: quantize_act -> linear (fp32 logits) ->
    verify_accept against 4 seeded uniform draft ids."""
    announce("tiny verify step")
    M, K, N, G = 5, 256, 512, 4
    bits = synth.activations_bf16(synth.W_TINY, M, K)
    w = synth.weights_f32(synth.W_TINY, N, K)
    draft = synth.draft_ids(synth.W_TINY, 1, G, N)
    xq_r, xs_r = oracle.quantize_act(bits)
    wq_r, ws_r = oracle.quantize_weight(w)
    acc_r, y32_r, y_r = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    am_r, al_r, nt_r = oracle.verify_accept(y32_r, draft)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wq, ws = w8.quantize_weight(dev(w))
    yb, yf, acc = w8.linear(xq, xs, wq, ws, want_bf16=True, want_f32=True, want_acc=True)
    am, al, nt = w8.verify_accept(yf, dev(draft))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), acc_r)
    np.testing.assert_array_equal(host(yb), y_r)
    np.testing.assert_array_equal(host(am), am_r)
    np.testing.assert_array_equal(host(al), al_r)
    np.testing.assert_array_equal(host(nt), nt_r)
