"""The Qwen3-32B-shaped linear stack at M = 8 (7 drafts + 1) on the GPU:
parity on sampled linears against the oracle.

The stack's weights are drawn on the GPU (synth.weights_device, torch's
device generator: 32 GB of N(0, 0.02) weights are too slow to draw on the
host).  For each sampled linear the same fp32 draw is copied to the host
and given to the oracle, which quantizes it itself; the GPU side quantizes
its device copy into the tiled layout.  Sampled: every linear of layers 0,
31 and 63, and the LM head 5120 -> 151936 with greedy acceptance of 7
drafts, two of which copy the oracle's argmax prefix.

Bars: int8 codes and scales, int32 accumulators and the fp32 dequant are
bit-exact; bf16 outputs bit-exact and within 1e-2 relative / 1e-3 absolute
of the oracle's fp32 dequant; argmax, accepted length and next token exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import announce, dev, dev_bf16, gpu_available, host

pytestmark = pytest.mark.gpu

M = 8
G = M - 1
LAYERS = (0, 31, 63)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no ROCm GPU")


def untile(t: np.ndarray, N: int, K: int) -> np.ndarray:
    tiles, steps = t.shape[0], t.shape[1]
    a = t.reshape(tiles, steps, 4, 16, 16).transpose(0, 3, 1, 2, 4)
    return a.reshape(tiles * 16, steps * 64)[:N, :K]


@pytest.mark.parametrize("layer", LAYERS)
@pytest.mark.parametrize("li", range(len(synth.QWEN3_32B_LAYER)))
def test_stack_linear(layer, li):
    import w8a8_quantized_verification_amd as w8
    lin = synth.QWEN3_32B_LAYER[li]
    announce(f"32B stack layer {layer} {lin.name} N={lin.N} K={lin.K}")
    wd = synth.weights_device(synth.W_STACK32B, synth.stack_tensor_index(layer, li),
                              lin.N, lin.K, "cuda:0")
    wt, ws = w8.quantize_weight(wd, tiled=True)
    w = host(wd)
    del wd
    bits = synth.activations_bf16(synth.W_STACK32B, M, lin.K,
                                  index=synth.stack_tensor_index(layer, li),
                                  outliers=True, layer=layer)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    yb, yf, acc = w8.linear(xq, xs, wt, ws, want_bf16=True, want_f32=True, want_acc=True)
    torch.cuda.synchronize()

    wq_r, ws_r = oracle.quantize_weight(w)
    del w
    xq_r, xs_r = oracle.quantize_act(bits)
    np.testing.assert_array_equal(host(ws).view(np.uint32), ws_r.view(np.uint32))
    np.testing.assert_array_equal(untile(host(wt), lin.N, lin.K), wq_r)
    np.testing.assert_array_equal(host(xq), xq_r)
    np.testing.assert_array_equal(host(xs).view(np.uint32), xs_r.view(np.uint32))
    acc_r, y32_r, y_r = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    np.testing.assert_array_equal(host(acc), acc_r)
    np.testing.assert_array_equal(host(yf).view(np.uint32), y32_r.view(np.uint32))
    np.testing.assert_array_equal(host(yb), y_r)
    y = oracle.bf16_to_f32(host(yb)).astype(np.float64)
    ref = y32_r.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 1e-3 + 1e-2 * np.abs(ref))


def test_stack_lm_head_verify():
    import w8a8_quantized_verification_amd as w8
    lin = synth.QWEN3_32B_LM_HEAD
    announce(f"32B stack LM head V={lin.N} K={lin.K}, {G} drafts")
    wd = synth.weights_device(synth.W_STACK32B,
                              synth.stack_tensor_index(synth.QWEN3_32B_LAYERS, 0),
                              lin.N, lin.K, "cuda:0")
    wt, ws = w8.quantize_weight(wd, tiled=True)
    w = host(wd)
    del wd
    wq_r, ws_r = oracle.quantize_weight(w)
    del w
    np.testing.assert_array_equal(host(ws).view(np.uint32), ws_r.view(np.uint32))
    rows = np.array([0, 1, 15, 16, lin.N - 1, 77777])
    np.testing.assert_array_equal(untile(host(wt), lin.N, lin.K)[rows], wq_r[rows])

    B = 3
    bits = synth.activations_bf16(synth.W_STACK32B, B * M, lin.K, index=900)
    xq_r, xs_r = oracle.quantize_act(bits)
    _, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    am_r = oracle.argmax_rows(y32_r).reshape(B, M)
    draft = synth.draft_ids(synth.W_STACK32B, B, G, lin.N, index=900)
    draft[1, :3] = am_r[1, :3]         # accepted length 3 unless the 4th draft also matches
    draft[2, :] = am_r[2, :G]          # every draft accepted
    am_r, al_r, nt_r = oracle.verify_accept(y32_r, draft)
    assert al_r[2] == G

    xq, xs = w8.quantize_act(dev_bf16(bits))
    d = dev(draft)
    lg, am, al, nt = w8.lm_head_verify(xq, xs, wt, ws, d, want_logits=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(xq), xq_r)
    np.testing.assert_array_equal(host(lg).view(np.uint32), y32_r.view(np.uint32))
    np.testing.assert_array_equal(host(am), am_r)
    np.testing.assert_array_equal(host(al), al_r)
    np.testing.assert_array_equal(host(nt), nt_r)
