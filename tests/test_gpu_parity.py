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
from tests.gpu_util import DEV, announce, dev, dev_bf16, gpu_available, host

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
              (3, 8208), (2, 131072),
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


@pytest.mark.parametrize("M,K", [(5, 4096), (288, 1024), (8, 25600)])
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

def untile(t: np.ndarray, N: int, K: int) -> np.ndarray:
    """Row-major [N][K] view of a tiled weight buffer [N/16][K/64][64][16]:
    lane l of (tile, step) holds channel 16*tile + l%16 and k = 64*step +
    16*(l//16) .. +15 (the layout stated in include/w8a8.h)."""
    tiles, steps = t.shape[0], t.shape[1]
    a = t.reshape(tiles, steps, 4, 16, 16)          # tile, step, k-group, channel, byte
    a = a.transpose(0, 3, 1, 2, 4)                  # tile, channel, step, k-group, byte
    return a.reshape(tiles * 16, steps * 64)[:N, :K]


def run_linear_case(M, N, K, seed, outliers=True, tiled=False):
    bits = synth.activations_bf16(seed, M, K, outliers=outliers and K > 0)
    w = synth.weights_f32(seed, N, K)
    xq_ref, xs_ref = oracle.quantize_act(bits)
    wq_ref, ws_ref = oracle.quantize_weight(w)
    acc_ref, y32_ref, y_ref = oracle.w8a8_linear(xq_ref, xs_ref, wq_ref, ws_ref)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wq, ws = w8.quantize_weight(dev(w), tiled=tiled)
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
    (8, 5120, 8192),      # Qwen3-32B o: 320 tiles, the 64 past the last round split four ways
    (8, 10240, 5120),     # Qwen3-32B q/k/v fused: 128 tail tiles split in two
    (7, 4100, 6144),      # one ragged tail tile split eight ways
    (1, 1000, 4096),      # one token, ragged N
    (16, 777, 1040),      # full 16-row tile, ragged N and a partial 64-wide K step
    (3, 17, 16),          # one 16-byte k group
    (5, 1, 4096),         # a single output channel
    (17, 300, 512),       # two row blocks
    (40, 257, 2048),      # three row blocks, ragged
    (5, 64, 0),           # empty contraction
]


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("M,N,K", LINEAR_CASES)
def test_linear(M, N, K, tiled):
    announce(f"linear M={M} N={N} K={K} tiled={tiled}")
    run_linear_case(M, N, K, seed=200 + M + N % 97 + K % 89, tiled=tiled)


@pytest.mark.parametrize("N,K", [(512, 256), (1000, 4096), (17, 25600), (33, 80), (5, 16)])
@pytest.mark.parametrize("smooth", [False, True])
def test_quantize_weight_tiled(N, K, smooth):
    """Tiled codes equal the oracle's row-major codes after un-tiling, every
    padding byte is zero, and tiling the row-major codes gives the same bytes."""
    announce(f"quantize_weight tiled N={N} K={K} smooth={smooth}")
    w = synth.weights_f32(104, N, K)
    s = synth.smoothing_vector(104, K) if smooth else None
    sd = None if s is None else dev(s)
    wt, ws = w8.quantize_weight(dev(w), sd, tiled=True)
    wr, _ = w8.quantize_weight(dev(w), sd)
    wt2 = w8.tile_weight(wr)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_weight(w, smooth=s)
    t = host(wt)
    assert t.shape == w8.tiled_shape(N, K)
    np.testing.assert_array_equal(untile(t, N, K), q_ref)
    np.testing.assert_array_equal(host(ws).view(np.uint32), s_ref.view(np.uint32))
    full = untile(t, t.shape[0] * 16, t.shape[1] * 64)
    pad = np.ones(full.shape, dtype=bool)
    pad[:N, :K] = False
    assert np.all(full[pad] == 0)
    np.testing.assert_array_equal(host(wt2), t)


@pytest.fixture
def forced_split(monkeypatch):
    """Force the cross-workgroup split-K path (a tuning override that must
    not change any result)."""
    monkeypatch.setenv("W8A8_SPLITK", "8")
    monkeypatch.setenv("W8A8_WAVES", "4")
    yield


@pytest.mark.parametrize("M,N,K", [(5, 1024, 4096), (8, 1000, 5120), (16, 17, 25600), (16, 96, 2048)])
@pytest.mark.parametrize("tiled", [False, True])
def test_linear_forced_split_k(M, N, K, tiled, forced_split):
    announce(f"linear forced split-K M={M} N={N} K={K} tiled={tiled}")
    assert w8.linear_workspace_bytes(M, N, K) > 0
    run_linear_case(M, N, K, seed=310 + N % 13, tiled=tiled)


def test_linear_narrow_output_splits_by_default():
    """An output of a single 16-channel tile with a long K takes the split-K
    path without any override."""
    announce("linear narrow output default split")
    assert w8.linear_workspace_bytes(5, 16, 25600) > 0
    run_linear_case(5, 16, 25600, seed=320, tiled=True)


def test_linear_outputs_subsets_and_workspace_reuse(forced_split):
    """Each output alone matches; repeated split-K calls on one workspace stay
    exact (the workspace is left zero-filled after every call)."""
    announce("linear output subsets + split-K workspace reuse")
    M, N, K = 5, 1024, 4096
    xq, xs, wq, ws = run_linear_case(M, N, K, seed=301, tiled=True)
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


@pytest.mark.parametrize("N,K", [(4096, 4096), (1024, 4096), (12288, 4096), (4096, 12288)])
@pytest.mark.parametrize("tiled", [True, False])
def test_linear_batched_m288(N, K, tiled):
    """Batched verification, M = 32 x (8+1) = 288, on every Qwen3-8B layer
    shape: the full int32, fp32 and bf16 results against the oracle."""
    announce(f"linear M=288 N={N} K={K} tiled={tiled}")
    run_linear_case(288, N, K, seed=302 + N % 7, tiled=tiled)


@pytest.mark.parametrize("M,N,K", [(17, 65, 80), (96, 64, 64), (97, 4099, 1040), (200, 130, 16),
                                   (513, 300, 2048), (97, 4099, 1024), (300, 8200, 2048),
                                   (513, 20000, 64), (200, 131072, 64), (100, 4096, 256),
                                   (33, 30000, 128), (288, 24600, 4096), (289, 131080, 1088)])
def test_linear_batched_ragged(M, N, K):
    """Ragged last tiles in M, N and K (tiled weights, row-major
    activations).  K a multiple of 64 sends wide grids to the LDS-pipelined
    kernels, which gather each 16-row activation fragment from the
    row-major rows (rows past M repeat the last row and are dropped):
    32 x 32 with 4, 3 or 2 stages and the 96-row form (N >= 8200 here),
    the 16 x 16 k-sliced form (4096 x 256); the rest take the register
    kernel."""
    announce(f"linear batched ragged M={M} N={N} K={K}")
    run_linear_case(M, N, K, seed=330 + M, tiled=True)


@pytest.mark.parametrize("M,N,K", [(288, 4096, 4096), (288, 1024, 4096), (288, 12288, 4096),
                                   (288, 4096, 12288), (17, 65, 80), (97, 4099, 1040),
                                   (513, 300, 2048), (5, 512, 256), (40, 33, 16), (288, 64, 0),
                                   (200, 20008, 1040), (513, 8200, 144), (288, 24576, 64),
                                   (200, 4000, 4096), (97, 4099, 1024), (288, 6144, 4096),
                                   (300, 6152, 2048), (65, 16384, 1040), (200, 131072, 64),
                                   (288, 24600, 4096), (288, 131080, 1040)])
def test_linear_tiled_activations(M, N, K):
    """quantize_act_tiled + linear_tiled_act: the codes read back through
    the tiled layout (padding zero) and every output against the oracle.
    Grids of 224+ workgroups of 64 rows x 128 channels (N >= 6144 here)
    take the 32 x 32 kernel with the weights streamed through registers:
    64 x 128 workgroups with 3 steps of lookahead below 768 such
    workgroups, 64 x 256 (two channel blocks per wave) from 768 (N = 24576,
    24600), 96 x 256 from 2048 96-row workgroups (N = 131072, 131080), with
    ragged row blocks, channel blocks (a wave's second block partly or
    wholly past N) and k steps (a step count that is not a multiple of the
    register ring); the 16 x 16 LDS kernel takes 128-511 of its own
    workgroups with a step count divisible by 4 (q, down and the ragged
    4000 / 4099-wide cases) in its k-sliced form; the rest the
    register-fragment kernel."""
    announce(f"linear tiled activations M={M} N={N} K={K}")
    seed = 340 + M + N % 11
    bits = synth.activations_bf16(seed, M, K, outliers=K > 0)
    w = synth.weights_f32(seed, N, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    wq_r, ws_r = oracle.quantize_weight(w)
    acc_r, y32_r, y_r = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    xt, xs = w8.quantize_act_tiled(dev_bf16(bits))
    wt, ws = w8.quantize_weight(dev(w), tiled=True)
    yb, yf, acc = w8.linear_tiled_act(xt, xs, wt, ws, K=K, want_bf16=True, want_f32=True,
                                      want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(xs).view(np.uint32), xs_r.view(np.uint32))
    if K > 0:
        t = host(xt)
        full = untile(t, t.shape[0] * 16, t.shape[1] * 64)
        np.testing.assert_array_equal(full[:M, :K], xq_r)
        assert not full[M:].any() and not full[:, K:].any()
    np.testing.assert_array_equal(host(acc), acc_r)
    np.testing.assert_array_equal(host(yf).view(np.uint32), y32_r.view(np.uint32))
    np.testing.assert_array_equal(host(yb), y_r)


@pytest.mark.parametrize("M,N,K,act,shift", [
    (288, 4096, 4096, "tiled", 0), (288, 6144, 4096, "tiled", 0), (288, 12288, 4096, "tiled", 0),
    (288, 24576, 4096, "tiled", 0), (288, 24600, 4096, "tiled", 0), (289, 6152, 1088, "tiled", 0),
    (288, 131080, 1040, "tiled", 0), (288, 4096, 4096, "rows", 0), (289, 6152, 1088, "rows", 0),
    (288, 6148, 1024, "tiled", 0), (288, 4096, 1024, "tiled", 1), (289, 6152, 1088, "rows", 1),
    (288, 4096, 12288, "tiled", 0), (288, 4096, 12288, "rows", 0), (280, 4000, 8208, "tiled", 0),
    (280, 4004, 8208, "tiled", 0), (288, 4096, 8192, "tiled", 1)])
def test_linear_bf16_only(M, N, K, act, shift):
    """Only the bf16 output requested, as in a model's layers: with N % 8 == 0
    and a 16-byte aligned output the 32 x 32 kernels store each 32 x 32 block
    through the wave's LDS tile as 16-byte row pieces (64 x 128, 64 x 256 and
    96 x 256 workgroups; ragged rows, channels and k steps; tiled and
    row-major activations); N % 8 != 0 or an output 2 bytes off alignment
    (shift = 1) take the element-wise epilogue.  From 128 k steps on the
    64 x 128 grids (K = 8192, 8208, 12288 at 4096 channels) the reduction is
    split across two workgroups (96 x 128 tiles, int32 partials handed over
    through the workspace) before either epilogue.  Every output against the
    oracle, bit for bit, and the 8 bf16 guard elements on either side of the
    output untouched."""
    announce(f"linear bf16-only M={M} N={N} K={K} act={act} shift={shift}")
    seed = 350 + M + N % 13 + K % 7
    bits = synth.activations_bf16(seed, M, K, outliers=True)
    w = synth.weights_f32(seed, N, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    wq_r, ws_r = oracle.quantize_weight(w)
    _, y32_r, y_r = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    wt, ws = w8.quantize_weight(dev(w), tiled=True)
    guard = 8 + shift
    flat = torch.full((M * N + 2 * guard,), -7.0, dtype=torch.bfloat16, device=DEV)
    y = flat[guard:guard + M * N].view(M, N)
    if act == "tiled":
        xt, xs = w8.quantize_act_tiled(dev_bf16(bits))
        w8.linear_tiled_act(xt, xs, wt, ws, K=K, want_bf16=False, y_bf16=y)
    else:
        xq, xs = w8.quantize_act(dev_bf16(bits))
        w8.linear(xq, xs, wt, ws, want_bf16=False, y_bf16=y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y), y_r)
    assert_bf16_tolerance(host(y), y32_r)
    f = host(flat).view(np.uint16)
    canary = host(torch.full((1,), -7.0, dtype=torch.bfloat16)).view(np.uint16)[0]
    assert (f[:guard] == canary).all() and (f[guard + M * N:] == canary).all()


def test_linear_split_workspace_shared():
    """One zero-filled workspace shared, in turn, by the batched kernel's k
    split (tiled and row-major activations, two shapes) and the skinny
    kernel's split-K (8 rows, 25600 -> 5120): each call against the oracle
    bit for bit, and the workspace zero-filled again after every call (the
    skinny split adds its partials onto whatever the buffer holds)."""
    announce("linear split workspace shared")
    wsp = w8.Workspace()
    cases = [(288, 4096, 12288, "tiled"), (8, 5120, 25600, "skinny"), (288, 4096, 12288, "rows"),
             (280, 4004, 8208, "tiled"), (8, 5120, 25600, "skinny"), (288, 4096, 12288, "tiled")]
    assert w8.linear_tiled_act_workspace_bytes(288, 4096, 12288) > 0
    assert w8.linear_workspace_bytes(288, 4096, 12288) > 0
    assert w8.linear_workspace_bytes(8, 5120, 25600) > 0
    for n, (M, N, K, kind) in enumerate(cases):
        announce(f"  call {n}: M={M} N={N} K={K} {kind}")
        seed = 370 + n
        bits = synth.activations_bf16(seed, M, K, outliers=True)
        w = synth.weights_f32(seed, N, K)
        xq_r, xs_r = oracle.quantize_act(bits)
        wq_r, ws_r = oracle.quantize_weight(w)
        acc_r, y32_r, y_r = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
        wt, ws = w8.quantize_weight(dev(w), tiled=True)
        if kind == "tiled":
            xt, xs = w8.quantize_act_tiled(dev_bf16(bits))
            yb, yf, acc = w8.linear_tiled_act(xt, xs, wt, ws, K=K, want_f32=True, want_acc=True,
                                              workspace=wsp)
        else:
            xq, xs = w8.quantize_act(dev_bf16(bits))
            yb, yf, acc = w8.linear(xq, xs, wt, ws, want_f32=True, want_acc=True, workspace=wsp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(acc), acc_r)
        np.testing.assert_array_equal(host(yf).view(np.uint32), y32_r.view(np.uint32))
        np.testing.assert_array_equal(host(yb), y_r)
        buf = wsp.get(1, torch.device(DEV), use="zeroed")
        assert not bool(buf.any()), f"call {n}: workspace not left zero-filled"


def test_linear_split_graph_replays():
    """The batched k split (288 x 4096 x 12288, tiled activations) captured
    in a HIP graph and replayed four times, with eager calls of another split
    shape and output clears between the replays: every replay against the
    oracle bit for bit (the arrival counters reset by each call, no memset
    in the graph), the workspace zero-filled after each."""
    announce("linear split graph replays")
    M, N, K = 288, 4096, 12288
    seed = 390
    bits = synth.activations_bf16(seed, M, K, outliers=True)
    w = synth.weights_f32(seed, N, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    wq_r, ws_r = oracle.quantize_weight(w)
    _, _, y_r = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    bits2 = synth.activations_bf16(seed + 1, 280, 8208, outliers=True)
    w2 = synth.weights_f32(seed + 1, 4004, 8208)
    xq2_r, xs2_r = oracle.quantize_act(bits2)
    wq2_r, ws2_r = oracle.quantize_weight(w2)
    _, _, y2_r = oracle.w8a8_linear(xq2_r, xs2_r, wq2_r, ws2_r)
    wsp = w8.Workspace()
    xt, xs = w8.quantize_act_tiled(dev_bf16(bits))
    wt, ws = w8.quantize_weight(dev(w), tiled=True)
    xt2, xs2 = w8.quantize_act_tiled(dev_bf16(bits2))
    wt2, ws2 = w8.quantize_weight(dev(w2), tiled=True)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    w8.linear_tiled_act(xt, xs, wt, ws, K=K, y_bf16=y, workspace=wsp)   # eager: allocates
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.linear_tiled_act(xt, xs, wt, ws, K=K, y_bf16=y, workspace=wsp)
    torch.cuda.synchronize()
    for r in range(4):
        y.zero_()
        y2, _, _ = w8.linear_tiled_act(xt2, xs2, wt2, ws2, K=8208, workspace=wsp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y2), y2_r)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), y_r)
        buf = wsp.get(1, torch.device(DEV), use="zeroed")
        assert not bool(buf.any()), f"replay {r}: workspace not left zero-filled"


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


def untile_bf16(t: np.ndarray, N: int, K: int) -> np.ndarray:
    """Row-major [N][K] view of a tiled bf16 weight [N/16][K/32][64][8]:
    lane l of (tile, step) holds channel 16*tile + l%16 and k = 32*step +
    8*(l//16) .. +7 (the layout stated in include/w8a8.h)."""
    tiles, steps = t.shape[0], t.shape[1]
    a = t.reshape(tiles, steps, 4, 16, 8)           # tile, step, k-group, channel, value
    a = a.transpose(0, 3, 1, 2, 4)                  # tile, channel, step, k-group, value
    return a.reshape(tiles * 16, steps * 32)


@pytest.mark.parametrize("M,N,K", [(5, 512, 256), (5, 4096, 4096), (8, 1000, 5120), (16, 33, 48),
                                   (5, 40000, 4096), (1, 32784, 1040), (3, 17, 4112)])
def test_bf16_reference_linear_tiled(M, N, K):
    """The tiled bf16 layout read back (every value in place, the padding
    zero) and the product on it against the float64 oracle within the
    summation-order bound, beside the row-major kernel's.  N >= 32768 takes
    two tiles per workgroup (32784: an odd tile count, the last
    workgroup's second tile past N); K = 1040, 4112 end in a half step."""
    announce(f"bf16 linear tiled M={M} N={N} K={K}")
    bits = synth.activations_bf16(510, M, K, outliers=True)
    w = synth.weights_f32(510, N, K)
    wb = synth.to_bf16_bits(w)
    ref = oracle.bf16_reference_logits(bits, w)
    wt = w8.tile_weight_bf16(dev_bf16(wb))
    full = untile_bf16(host(wt), N, K)
    np.testing.assert_array_equal(full[:N, :K], wb)
    assert not full[N:].any() and not full[:, K:].any()
    yb, yf = w8.bf16_linear(dev_bf16(bits), wt, N=N, want_bf16=True, want_f32=True)
    _, yf_rm = w8.bf16_linear(dev_bf16(bits), dev_bf16(wb), want_bf16=False, want_f32=True)
    torch.cuda.synchronize()
    x64 = np.abs(oracle.bf16_to_f32(bits).astype(np.float64))
    w64 = np.abs(oracle.bf16_to_f32(wb).astype(np.float64))
    bound = K * 2.0 ** -23 * (x64 @ w64.T)
    assert np.all(np.abs(host(yf).astype(np.float64) - ref) <= bound)
    assert np.all(np.abs(host(yf_rm).astype(np.float64) - ref) <= bound)
    np.testing.assert_array_equal(host(yb), oracle.f32_to_bf16(host(yf)))


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


# --------------------------------------------------------------------------
# the step captured in a HIP graph (the benchmark replays it this way)
# --------------------------------------------------------------------------

def test_graph_replay_matches_eager(forced_split):
    """A verify step (quantize_act, a split-K linear, the LM-head-style linear
    and verify_accept) captured once in a HIP graph: every replay, with eager
    work and synchronizations between replays, equals the eager result."""
    announce("graph replay of a verify step")
    M, K, Nmid, V, G = 5, 4096, 1024, 4099, 4
    bits = synth.activations_bf16(600, M, K)
    w1 = synth.weights_f32(600, Nmid, K)
    w2 = synth.weights_f32(601, V, K)
    x = dev_bf16(bits)
    wq1, ws1 = w8.quantize_weight(dev(w1), tiled=True)
    wq2, ws2 = w8.quantize_weight(dev(w2), tiled=True)
    draft = dev(synth.draft_ids(600, 1, G, V))
    assert w8.linear_workspace_bytes(M, Nmid, K) > 0  # the split-K path is in the graph
    ws = w8.Workspace()
    xq = torch.empty(M, K, dtype=torch.int8, device="cuda:0")
    xs = torch.empty(M, dtype=torch.float32, device="cuda:0")
    mid = torch.empty(M, Nmid, dtype=torch.int32, device="cuda:0")
    lg = torch.empty(M, V, dtype=torch.float32, device="cuda:0")
    am = torch.empty(M, dtype=torch.int32, device="cuda:0")
    al = torch.empty(1, dtype=torch.int32, device="cuda:0")
    nt = torch.empty(1, dtype=torch.int32, device="cuda:0")

    am2 = torch.empty(M, dtype=torch.int32, device="cuda:0")
    al2 = torch.empty(1, dtype=torch.int32, device="cuda:0")
    nt2 = torch.empty(1, dtype=torch.int32, device="cuda:0")

    def step():
        w8.quantize_act(x, xq=xq, x_scale=xs)
        w8.linear(xq, xs, wq1, ws1, want_bf16=False, acc=mid, workspace=ws)
        w8.linear(xq, xs, wq2, ws2, want_bf16=False, y_f32=lg, workspace=ws)
        w8.verify_accept(lg, draft, argmax=am, accept_len=al, next_token=nt, workspace=ws)
        w8.lm_head_verify(xq, xs, wq2, ws2, draft, argmax=am2, accept_len=al2, next_token=nt2,
                          workspace=ws)

    outs = (xq, xs, mid, lg, am, al, nt, am2, al2, nt2)
    step()
    torch.cuda.synchronize()
    ref = [host(t) for t in outs]
    np.testing.assert_array_equal(ref[7], ref[4])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(5):
        for t in outs:
            t.zero_()
        scratch = torch.randn(1 << 20, device="cuda:0").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(t) for t in outs]
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {r}")
        del scratch


def test_graph_replay_split_tail():
    """The skinny kernel's split tail (8 x 8192 -> 5120: 320 tiles on 256
    CUs, the 64 past the last whole round cut into 4 k slices with the
    atomic hand-off) and a narrow split-K linear in one HIP graph: each
    replay equals the eager result and leaves the workspace zero."""
    announce("graph replay of the split tail")
    gen = torch.Generator(device="cuda:0").manual_seed(613)
    M, K, N, N2, K2 = 8, 8192, 5120, 512, 25600
    assert w8.linear_workspace_bytes(M, N, K) > 0 and w8.linear_workspace_bytes(M, N2, K2) > 0
    x = (torch.randn(M, K, device="cuda:0", generator=gen)).to(torch.bfloat16)
    x2 = (torch.randn(M, K2, device="cuda:0", generator=gen)).to(torch.bfloat16)
    wq, wsc = w8.quantize_weight(torch.randn(N, K, device="cuda:0", generator=gen) * 0.02, tiled=True)
    wq2, wsc2 = w8.quantize_weight(torch.randn(N2, K2, device="cuda:0", generator=gen) * 0.02,
                                   tiled=True)
    xq, xs = w8.quantize_act(x)
    xq2, xs2 = w8.quantize_act(x2)
    ws = w8.Workspace()
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda:0")
    acc = torch.empty(M, N, dtype=torch.int32, device="cuda:0")
    y2 = torch.empty(M, N2, dtype=torch.bfloat16, device="cuda:0")

    def step():
        w8.linear(xq, xs, wq, wsc, y_bf16=y, acc=acc, workspace=ws)
        w8.linear(xq2, xs2, wq2, wsc2, y_bf16=y2, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [host(t) for t in (y, acc, y2)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for t in (y, acc, y2):
            t.zero_()
        scratch = torch.randn(1 << 20, device="cuda:0").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((host(t) for t in (y, acc, y2)), ref):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {r}")
        assert not bool(ws.get(1, torch.device("cuda:0"), "zeroed").any()), f"replay {r}"
        del scratch


def test_graph_replay_batched_and_stochastic_steps():
    """The 288-row verify step (quantize_act_tiled; the down-shaped linear
    12288 -> 4096, whose k is split across two workgroups through the zeroed
    workspace; the LM-head argmax on tiled activations in its 96 x 256 form;
    accept_from_keys) and a T = 1 step (the LM-head linear to fp32 logits,
    then verify_sample's three kernels) captured in one HIP graph: every
    replay, with eager work and synchronizations between replays, equals the
    eager result bit for bit, and the zero-on-exit workspaces are zero after
    each replay."""
    announce("graph replay of the 288-row and T = 1 steps")
    gen = torch.Generator(device="cuda:0").manual_seed(612)
    M, Kd, Nd, K, V, B, G = 288, 12288, 4096, 4096, 100003, 32, 8

    def randn(*shape, scale=1.0):
        return torch.randn(*shape, device="cuda:0", generator=gen) * scale

    xd = randn(M, Kd).to(torch.bfloat16)
    x = randn(M, K).to(torch.bfloat16)
    wq_d, ws_d = w8.quantize_weight(randn(Nd, Kd, scale=0.02), tiled=True)
    wq_v, ws_v = w8.quantize_weight(randn(V, K, scale=0.02), tiled=True)
    assert w8.linear_tiled_act_workspace_bytes(M, Nd, Kd) > 0   # the k split is in the graph
    draft = torch.randint(0, V, (B, G), device="cuda:0", generator=gen, dtype=torch.int32)
    d5 = draft[:1, :4].contiguous()
    ua = torch.randint(-(1 << 31), 1 << 31, (1, 4), device="cuda:0", generator=gen, dtype=torch.int64)
    ua = ua.to(torch.int32)
    us = torch.randint(-(1 << 62), 1 << 62, (1,), device="cuda:0", generator=gen, dtype=torch.int64)
    ws = w8.Workspace()
    xt_d = torch.empty(w8.tiled_shape(M, Kd), dtype=torch.int8, device="cuda:0")
    xs_d = torch.empty(M, dtype=torch.float32, device="cuda:0")
    xt = torch.empty(w8.tiled_shape(M, K), dtype=torch.int8, device="cuda:0")
    xs = torch.empty(M, dtype=torch.float32, device="cuda:0")
    yd = torch.empty(M, Nd, dtype=torch.bfloat16, device="cuda:0")
    am = torch.empty(M, dtype=torch.int32, device="cuda:0")
    al = torch.empty(B, dtype=torch.int32, device="cuda:0")
    nt = torch.empty(B, dtype=torch.int32, device="cuda:0")
    xq5 = torch.empty(5, K, dtype=torch.int8, device="cuda:0")
    xs5 = torch.empty(5, dtype=torch.float32, device="cuda:0")
    lg5 = torch.empty(5, V, dtype=torch.float32, device="cuda:0")
    al5 = torch.empty(1, dtype=torch.int32, device="cuda:0")
    nt5 = torch.empty(1, dtype=torch.int32, device="cuda:0")

    def step():
        w8.quantize_act_tiled(xd, xq_tiled=xt_d, x_scale=xs_d)
        w8.linear_tiled_act(xt_d, xs_d, wq_d, ws_d, K=Kd, y_bf16=yd, workspace=ws)
        w8.quantize_act_tiled(x, xq_tiled=xt, x_scale=xs)
        w8.lm_head_argmax_tiled_act(xt, xs, wq_v, ws_v, K=K, workspace=ws)
        w8.accept_from_keys(draft, argmax=am, accept_len=al, next_token=nt, workspace=ws)
        w8.quantize_act(x[:5], xq=xq5, x_scale=xs5)
        w8.linear(xq5, xs5, wq_v, ws_v, want_bf16=False, y_f32=lg5, workspace=ws)
        w8.verify_sample(lg5, d5, 1.0, ua, us, accept_len=al5, next_token=nt5, workspace=ws)

    outs = (xt_d, xs_d, yd, xt, xs, am, al, nt, xq5, xs5, lg5, al5, nt5)
    step()
    torch.cuda.synchronize()
    ref = [host(t) for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for t in outs:
            t.zero_()
        scratch = torch.randn(1 << 20, device="cuda:0").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((host(t) for t in outs), ref):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {r}")
        for use in ("zeroed", "keys"):
            buf = ws.get(1, torch.device("cuda:0"), use)      # the buffer the step used
            assert not bool(buf.any()), f"workspace '{use}' not zero after replay {r}"
        del scratch


# --------------------------------------------------------------------------
# fused LM-head verification
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,G,V,K", [(1, 4, 512, 256), (1, 4, 151936, 4096), (32, 8, 4099, 1024),
                                     (1, 7, 5000, 5120), (3, 0, 1000, 256), (2, 3, 17, 64),
                                     (1, 15, 40000, 2048), (8, 1, 3000, 512), (4, 3, 20000, 1024),
                                     (3, 5, 9000, 256)])
def test_lm_head_verify(B, G, V, K):
    """Fused LM-head linear + argmax + acceptance against the oracle and
    against the separate linear -> verify_accept path."""
    announce(f"lm_head_verify B={B} G={G} V={V} K={K}")
    R = B * (G + 1)
    bits = synth.activations_bf16(700, R, K)
    w = synth.weights_f32(700, V, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    wq_r, ws_r = oracle.quantize_weight(w)
    _, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    am_r = oracle.argmax_rows(y32_r).reshape(B, G + 1)
    draft = synth.draft_ids(700, B, G, V)
    for b in range(B):                       # spread the accepted lengths
        p = b % (G + 1)
        draft[b, :p] = am_r[b, :p]
    am_r, al_r, nt_r = oracle.verify_accept(y32_r, draft)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wt, ws = w8.quantize_weight(dev(w), tiled=True)
    d = dev(draft)
    lg, am, al, nt = w8.lm_head_verify(xq, xs, wt, ws, d, want_logits=True)
    _, am2, al2, nt2 = w8.lm_head_verify(xq, xs, wt, ws, d)          # no logits written
    _, yf, _ = w8.linear(xq, xs, wt, ws, want_bf16=False, want_f32=True)
    am3, al3, nt3 = w8.verify_accept(yf, d)
    lg4 = w8.lm_head_argmax(xq, xs, wt, ws, logits=torch.empty_like(yf))   # the two phases
    am4, al4, nt4 = w8.accept_from_keys(d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(lg).view(np.uint32), y32_r.view(np.uint32))
    np.testing.assert_array_equal(host(lg4).view(np.uint32), y32_r.view(np.uint32))
    for a, l, n in ((am, al, nt), (am2, al2, nt2), (am3, al3, nt3), (am4, al4, nt4)):
        np.testing.assert_array_equal(host(a), am_r)
        np.testing.assert_array_equal(host(l), al_r)
        np.testing.assert_array_equal(host(n), nt_r)


@pytest.mark.parametrize("B,G,V,K", [(1, 4, 151936, 4096), (2, 7, 5000, 256), (16, 0, 4099, 128),
                                     (1, 0, 64, 64)])
def test_lm_head_verify_repeats_leave_workspace_zeroed(B, G, V, K):
    """Three calls in a row on one workspace (different drafts and hidden
    states) each match the two-phase path and the oracle, and leave the
    workspace (the argmax keys) zero-filled for the next call."""
    announce(f"lm_head_verify repeats B={B} G={G} V={V} K={K}")
    R = B * (G + 1)
    w = synth.weights_f32(710, V, K)
    wq_r, ws_r = oracle.quantize_weight(w)
    wt, ws = w8.quantize_weight(dev(w), tiled=True)
    wsp = w8.Workspace()
    for call in range(3):
        bits = synth.activations_bf16(711 + call, R, K)
        xq_r, xs_r = oracle.quantize_act(bits)
        _, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
        draft = synth.draft_ids(712 + call, B, G, V)
        am0 = oracle.argmax_rows(y32_r).reshape(B, G + 1)
        for b in range(B):
            p = (b + call) % (G + 1)
            draft[b, :p] = am0[b, :p]
        am_r, al_r, nt_r = oracle.verify_accept(y32_r, draft)
        xq, xs = w8.quantize_act(dev_bf16(bits))
        d = dev(draft)
        _, am, al, nt = w8.lm_head_verify(xq, xs, wt, ws, d, workspace=wsp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(am), am_r)
        np.testing.assert_array_equal(host(al), al_r)
        np.testing.assert_array_equal(host(nt), nt_r)
        buf = wsp.get(1, xq.device, use="keys")
        assert not bool(buf.any()), "workspace not left zero-filled"
        w8.lm_head_argmax(xq, xs, wt, ws, workspace=wsp)                 # the two phases
        am2, al2, nt2 = w8.accept_from_keys(d, workspace=wsp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(am2), am_r)
        np.testing.assert_array_equal(host(al2), al_r)
        np.testing.assert_array_equal(host(nt2), nt_r)


def test_lm_head_verify_ties_across_workgroups():
    """Equal maxima in columns owned by different workgroups (and inside one
    16-column tile): the lowest index wins."""
    announce("lm_head_verify ties")
    M, K, V = 5, 64, 4096
    hot = {0: [100, 3000], 1: [5, 7], 2: [4095, 2048, 64], 3: [0, 4095], 4: [31, 32, 33]}
    # row r reads only k = r, where exactly its hot columns hold a weight
    xq = torch.zeros(M, K, dtype=torch.int8, device="cuda:0")
    wq = torch.zeros(V, K, dtype=torch.int8, device="cuda:0")
    for r, cols in hot.items():
        xq[r, r] = 1
        for c in cols:
            wq[c, r] = 3
    xs = torch.ones(M, dtype=torch.float32, device="cuda:0")
    ws = torch.ones(V, dtype=torch.float32, device="cuda:0")
    wt = w8.tile_weight(wq)
    draft = torch.tensor([[100, 5, 64, 0]], dtype=torch.int32, device="cuda:0")
    _, am, al, nt = w8.lm_head_verify(xq, xs, wt, ws, draft)
    torch.cuda.synchronize()
    assert host(am).tolist() == [100, 5, 64, 0, 31]
    assert int(host(al)[0]) == 4 and int(host(nt)[0]) == 31


def test_lm_head_argmax_timed_matches_and_times():
    """The launch that records the kernel's own timestamps into two events
    gives the same keys (acceptance) as the plain launch, and a positive
    duration for each call."""
    announce("lm_head_argmax timed")
    B, G, V, K = 1, 4, 151936, 4096
    R = B * (G + 1)
    bits = synth.activations_bf16(740, R, K)
    w = synth.weights_f32(740, V, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    wq_r, ws_r = oracle.quantize_weight(w)
    _, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    draft = synth.draft_ids(740, B, G, V)
    draft[0, :2] = oracle.argmax_rows(y32_r)[:2]
    am_r, al_r, nt_r = oracle.verify_accept(y32_r, draft)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wt, ws = w8.quantize_weight(dev(w), tiled=True)
    d = dev(draft)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(3)]
    for a, b in evs:                 # torch creates the events on their first record
        a.record()
        b.record()
    for e in evs:
        lg = w8.lm_head_argmax(xq, xs, wt, ws, logits=torch.empty(R, V, dtype=torch.float32,
                                                                  device=xq.device), events=e)
        am, al, nt = w8.accept_from_keys(d)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(lg).view(np.uint32), y32_r.view(np.uint32))
        np.testing.assert_array_equal(host(am), am_r)
        np.testing.assert_array_equal(host(al), al_r)
        np.testing.assert_array_equal(host(nt), nt_r)
        t = e[0].elapsed_time(e[1])
        assert 0.0 < t < 100.0, t


# --------------------------------------------------------------------------
# batched LM-head verification with tiled activations
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,G,V,K", [(32, 8, 151936, 4096), (32, 8, 4099, 1024), (32, 8, 20000, 256),
                                     (7, 8, 12000, 1040), (30, 8, 16384, 64), (25, 8, 8200, 2048),
                                     (1, 4, 40000, 256), (30, 8, 100000, 256)])
def test_lm_head_argmax_tiled_act(B, G, V, K):
    """quantize_act_tiled -> lm_head_argmax_tiled_act -> accept_from_keys
    for many verified rows: logits, argmax and acceptance against the oracle
    and against the row-major lm_head_argmax (the wide grids take the
    32 x 32 MFMA kernel with the argmax folded in: 96-row workgroups for 288
    rows over the full vocabulary and for the 100000-wide case, 64-row ones
    with 2-4 stages for the others from 20000 channels up; the narrower
    grids the register-fragment kernel)."""
    announce(f"lm_head_argmax_tiled_act B={B} G={G} V={V} K={K}")
    R = B * (G + 1)
    bits = synth.activations_bf16(760, R, K)
    w = synth.weights_f32(760, V, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    wq_r, ws_r = oracle.quantize_weight(w)
    _, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    am_r = oracle.argmax_rows(y32_r).reshape(B, G + 1)
    draft = synth.draft_ids(760, B, G, V)
    for b in range(B):
        p = b % (G + 1)
        draft[b, :p] = am_r[b, :p]
    am_r, al_r, nt_r = oracle.verify_accept(y32_r, draft)
    x = dev_bf16(bits)
    xt, xs = w8.quantize_act_tiled(x)
    wt, ws = w8.quantize_weight(dev(w), tiled=True)
    d = dev(draft)
    wsp = w8.Workspace()
    lg = w8.lm_head_argmax_tiled_act(xt, xs, wt, ws, K=K, workspace=wsp,
                                     logits=torch.empty(R, V, dtype=torch.float32, device=x.device))
    am, al, nt = w8.accept_from_keys(d, workspace=wsp)
    w8.lm_head_argmax_tiled_act(xt, xs, wt, ws, K=K, workspace=wsp)        # no logits
    am2, al2, nt2 = w8.accept_from_keys(d, workspace=wsp)
    xq, xs3 = w8.quantize_act(x)
    w8.lm_head_argmax(xq, xs3, wt, ws, workspace=wsp)
    am3, al3, nt3 = w8.accept_from_keys(d, workspace=wsp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(lg).view(np.uint32), y32_r.view(np.uint32))
    for a, l, n in ((am, al, nt), (am2, al2, nt2), (am3, al3, nt3)):
        np.testing.assert_array_equal(host(a), am_r)
        np.testing.assert_array_equal(host(l), al_r)
        np.testing.assert_array_equal(host(n), nt_r)
    assert not bool(wsp.get(1, x.device, use="keys").any())


def test_lm_head_argmax_tiled_act_ties():
    """Equal maxima in different 32-channel blocks, workgroups and inside one
    block, on a grid wide enough for the 32 x 32 kernel: the lowest index
    wins."""
    announce("lm_head_argmax_tiled_act ties")
    M, K, V = 5, 64, 32768
    hot = {0: [100, 3000], 1: [5, 7], 2: [32767, 16384, 64], 3: [0, 32767], 4: [31, 32, 33]}
    xq = torch.zeros(M, K, dtype=torch.int8, device="cuda:0")
    wq = torch.zeros(V, K, dtype=torch.int8, device="cuda:0")
    for r, cols in hot.items():
        xq[r, r] = 1
        for c in cols:
            wq[c, r] = 3
    xs = torch.ones(M, dtype=torch.float32, device="cuda:0")
    ws = torch.ones(V, dtype=torch.float32, device="cuda:0")
    wt = w8.tile_weight(wq)
    xt = w8.tile_weight(xq)            # the same tiled layout, token rows as channels
    draft = torch.tensor([[100, 5, 64, 0]], dtype=torch.int32, device="cuda:0")
    w8.lm_head_argmax_tiled_act(xt, xs, wt, ws, K=K)
    am, al, nt = w8.accept_from_keys(draft)
    torch.cuda.synchronize()
    assert host(am).tolist() == [100, 5, 64, 0, 31]
    assert int(host(al)[0]) == 4 and int(host(nt)[0]) == 31


def test_lm_head_argmax_ties_96_row_workgroups():
    """Ties on the grid that takes the 96-row 32 x 32 workgroups (288 rows,
    100000 channels): each row reads one k, whose equal maxima sit in one
    32-channel block, in adjacent blocks, in different workgroups and in the
    last (partial) tile; the lowest index wins for tiled and row-major
    activations alike."""
    announce("lm_head_argmax ties, 96-row workgroups")
    M, K, V = 288, 64, 100000
    xq = torch.zeros(M, K, dtype=torch.int8, device="cuda:0")
    wq = torch.zeros(V, K, dtype=torch.int8, device="cuda:0")
    expect = []
    for k in range(K):
        base = (k * 1543) % (V - 64)
        cols = {base + 31, base + 32, (k * 7919 + 50000) % V, V - 1 - k, base + 33}
        for c in cols:
            wq[c, k] = 3
        expect.append(min(cols))
    rows = np.arange(M) % K
    xq[torch.arange(M, device="cuda:0"), torch.from_numpy(rows).long().to("cuda:0")] = 1
    xs = torch.ones(M, dtype=torch.float32, device="cuda:0")
    ws = torch.ones(V, dtype=torch.float32, device="cuda:0")
    wt = w8.tile_weight(wq)
    xt = w8.tile_weight(xq)            # the same tiled layout, token rows as channels
    B, G = 32, 8
    want = np.array([expect[r] for r in rows], dtype=np.int32)
    draft = torch.from_numpy(want.reshape(B, G + 1)[:, :G].copy()).to("cuda:0")
    for tiled_act in (True, False):
        if tiled_act:
            w8.lm_head_argmax_tiled_act(xt, xs, wt, ws, K=K)
        else:
            w8.lm_head_argmax(xq, xs, wt, ws)
        am, al, nt = w8.accept_from_keys(draft)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(am), want)
        assert host(al).tolist() == [G] * B
        np.testing.assert_array_equal(host(nt), want.reshape(B, G + 1)[:, G])
