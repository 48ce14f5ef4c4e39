"""GPU parity of the chained verify step (w8a8_chain_*: one persistent launch
for a sequence of quantize / linear / LM-head / accept steps) against the
CPU oracle, through the C ABI.

Bars as for the separate calls: int8 codes, scales, fp32 dequant, bf16
outputs, argmax, accepted lengths and next tokens bit-exact.  The chains
here make every step read what the step before it wrote (bf16 output ->
quantization -> next linear), so a missing or leaky barrier shows up as a
wrong code; runs are repeated, replayed from a HIP graph and checked for a
clean status.
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


def _weights(seed, N, K):
    """fp32 weights, the oracle's codes/scales and the device tiled codes."""
    w = synth.weights_f32(seed, N, K)
    wq_r, ws_r = oracle.quantize_weight(w)
    wt, ws = w8.quantize_weight(dev(w), tiled=True)
    return (wq_r, ws_r), (wt, ws)


def _dependent_chain(M, dims, seed, smooth=False):
    """x[M][dims[0]] -> quantize -> linear to dims[1] -> quantize -> linear to
    dims[2] ... ; returns (chain, device outputs, oracle outputs)."""
    bits = synth.activations_bf16(seed, M, dims[0], outliers=True)
    x = dev_bf16(bits)
    sm = synth.smoothing_vector(seed, dims[0]) if smooth else None
    steps, outs, ref = [], [], []
    cur_dev, cur_bits = x, bits
    for i in range(len(dims) - 1):
        K, N = dims[i], dims[i + 1]
        xq = torch.empty(M, K, dtype=torch.int8, device=x.device)
        xs = torch.empty(M, dtype=torch.float32, device=x.device)
        s_dev = dev(sm) if (sm is not None and i == 0) else None
        steps.append(w8.chain_quantize(cur_dev, xq=xq, x_scale=xs, smooth=s_dev))
        (wq_r, ws_r), (wt, ws) = _weights(seed + 10 + i, N, K)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
        y32 = torch.empty(M, N, dtype=torch.float32, device=x.device)
        steps.append(w8.chain_linear(xq, xs, wt, ws, y_bf16=y, y_f32=y32))
        q_r, s_r = oracle.quantize_act(cur_bits, sm if i == 0 else None)
        _, y32_r, y_r = oracle.w8a8_linear(q_r, s_r, wq_r, ws_r)
        outs.append((xq, xs, y, y32))
        ref.append((q_r, s_r, y_r, y32_r))
        cur_dev, cur_bits = y, y_r
    return w8.Chain(steps), outs, ref


def _check(outs, ref):
    for i, ((xq, xs, y, y32), (q_r, s_r, y_r, y32_r)) in enumerate(zip(outs, ref)):
        np.testing.assert_array_equal(host(xq), q_r, err_msg=f"codes of step {2 * i}")
        np.testing.assert_array_equal(host(xs).view(np.uint32), s_r.view(np.uint32))
        np.testing.assert_array_equal(host(y32).view(np.uint32), y32_r.view(np.uint32),
                                      err_msg=f"y32 of step {2 * i + 1}")
        np.testing.assert_array_equal(host(y), y_r)


# widths: several tiles, K not a multiple of 64 (4112), a ragged last N
DEP_CASES = [(5, (4096, 1040, 4112, 777)), (1, (256, 16, 64, 33)), (16, (2048, 3072, 1008)),
             (8, (5120, 1024, 25600, 5120)), (3, (12288, 4096, 4096))]


@pytest.mark.parametrize("M,dims", DEP_CASES)
def test_chain_dependent_steps(M, dims):
    announce(f"chain dependent M={M} dims={dims}")
    ch, outs, ref = _dependent_chain(M, dims, 900 + M)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    _check(outs, ref)


def test_chain_smoothing():
    announce("chain quantize with smoothing")
    ch, outs, ref = _dependent_chain(5, (4096, 2048, 512), 950, smooth=True)
    ch.run()
    assert ch.status() == 0
    _check(outs, ref)


def test_chain_matches_separate_calls():
    """The Qwen3-8B layer's four fused linears at M = 5 with their input
    quantizations, as one chain, equal the separate calls bit for bit."""
    announce("chain vs separate calls, Qwen3-8B layer shapes M=5")
    M = 5
    shapes = ((6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288))
    steps, got, want = [], [], []
    for i, (N, K) in enumerate(shapes):
        x = dev_bf16(synth.activations_bf16(960 + i, M, K, outliers=True))
        wt, ws = w8.quantize_weight(dev(synth.weights_f32(970 + i, N, K)), tiled=True)
        xq = torch.empty(M, K, dtype=torch.int8, device=x.device)
        xs = torch.empty(M, dtype=torch.float32, device=x.device)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
        steps += [w8.chain_quantize(x, xq=xq, x_scale=xs),
                  w8.chain_linear(xq, xs, wt, ws, y_bf16=y)]
        q2, s2 = w8.quantize_act(x)
        y2, _, _ = w8.linear(q2, s2, wt, ws)
        got.append((xq, xs, y))
        want.append((q2, s2, y2))
    ch = w8.Chain(steps)
    ch.run()
    assert ch.status() == 0
    for (a, b, c), (a2, b2, c2) in zip(got, want):
        assert torch.equal(a, a2) and torch.equal(b, b2)
        assert torch.equal(c.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("B,G,V,K", [(1, 4, 151936, 4096), (2, 7, 4099, 1024), (3, 0, 1000, 256),
                                     (1, 15, 40000, 2048), (4, 3, 17, 64), (1, 7, 151936, 5120),
                                     (1, 4, 64, 16384)])
def test_chain_lm_head_accept(B, G, V, K):
    """quantize -> LM head with the argmax fold -> acceptance in one chain,
    against the oracle, with the accepted lengths spread over 0..G (the
    last case: four tiles over a long K, split across workgroups)."""
    announce(f"chain lm head B={B} G={G} V={V} K={K}")
    M = B * (G + 1)
    bits = synth.activations_bf16(980, M, K)
    (wq_r, ws_r), (wt, ws) = _weights(981, V, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    _, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    am0 = oracle.argmax_rows(y32_r).reshape(B, G + 1)
    draft = synth.draft_ids(982, B, G, V)
    for b in range(B):
        p = b % (G + 1)
        draft[b, :p] = am0[b, :p]
    am_r, al_r, nt_r = oracle.verify_accept(y32_r, draft)
    x = dev_bf16(bits)
    xq = torch.empty(M, K, dtype=torch.int8, device=x.device)
    xs = torch.empty(M, dtype=torch.float32, device=x.device)
    lg = torch.empty(M, V, dtype=torch.float32, device=x.device)
    am = torch.empty(M, dtype=torch.int32, device=x.device)
    al = torch.empty(B, dtype=torch.int32, device=x.device)
    nt = torch.empty(B, dtype=torch.int32, device=x.device)
    d = dev(draft)
    ch = w8.Chain([w8.chain_quantize(x, xq=xq, x_scale=xs),
                   w8.chain_lm_head(xq, xs, wt, ws, logits=lg),
                   w8.chain_accept(d, argmax=am, accept_len=al, next_token=nt)])
    for rep in range(3):     # the keys are reset by every ACCEPT
        am.fill_(-1)
        al.fill_(-1)
        ch.run()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(lg).view(np.uint32), y32_r.view(np.uint32))
        np.testing.assert_array_equal(host(am), am_r)
        np.testing.assert_array_equal(host(al), al_r)
        np.testing.assert_array_equal(host(nt), nt_r)
    assert ch.status() == 0


def test_chain_two_lm_heads():
    """Two LM_HEAD/ACCEPT pairs in one chain (different heads, the second
    without logits): each verdict equals the oracle's."""
    announce("chain two lm heads")
    B, G, K = 1, 4, 1024
    M = B * (G + 1)
    bits = synth.activations_bf16(990, M, K)
    x = dev_bf16(bits)
    xq = torch.empty(M, K, dtype=torch.int8, device=x.device)
    xs = torch.empty(M, dtype=torch.float32, device=x.device)
    steps, outs, refs = [w8.chain_quantize(x, xq=xq, x_scale=xs)], [], []
    xq_r, xs_r = oracle.quantize_act(bits)
    for j, V in enumerate((5003, 30000)):
        (wq_r, ws_r), (wt, ws) = _weights(991 + j, V, K)
        _, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
        draft = synth.draft_ids(993 + j, B, G, V)
        draft[0, :2 + j] = oracle.argmax_rows(y32_r)[:2 + j]
        refs.append(oracle.verify_accept(y32_r, draft))
        o = [torch.empty(M, dtype=torch.int32, device=x.device)] + \
            [torch.empty(B, dtype=torch.int32, device=x.device) for _ in range(2)]
        steps += [w8.chain_lm_head(xq, xs, wt, ws),
                  w8.chain_accept(dev(draft), argmax=o[0], accept_len=o[1], next_token=o[2])]
        outs.append(o)
    ch = w8.Chain(steps)
    ch.run()
    assert ch.status() == 0
    for o, r in zip(outs, refs):
        for a, b in zip(o, r):
            np.testing.assert_array_equal(host(a), b)


@pytest.mark.parametrize("M,N,K", [(1, 16, 64), (4, 32, 8192), (8, 5120, 25600), (16, 48, 16),
                                   (2, 100000, 64), (7, 3000, 4160)])
def test_chain_linear_shapes(M, N, K):
    """Stream-K edge cases: one block in all, many contributors per tile
    (2 tiles x 128 steps), long K, K = 16, many one-step tiles, ragged N."""
    announce(f"chain linear M={M} N={N} K={K}")
    bits = synth.activations_bf16(1000 + K, M, K, outliers=True)
    (wq_r, ws_r), (wt, ws) = _weights(1001, N, K)
    q_r, s_r = oracle.quantize_act(bits)
    _, y32_r, y_r = oracle.w8a8_linear(q_r, s_r, wq_r, ws_r)
    x = dev_bf16(bits)
    xq = torch.empty(M, K, dtype=torch.int8, device=x.device)
    xs = torch.empty(M, dtype=torch.float32, device=x.device)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
    y32 = torch.empty(M, N, dtype=torch.float32, device=x.device)
    ch = w8.Chain([w8.chain_quantize(x, xq=xq, x_scale=xs),
                   w8.chain_linear(xq, xs, wt, ws, y_bf16=y, y_f32=y32)])
    for _ in range(2):
        y32.zero_()
        ch.run()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(xq), q_r)
        np.testing.assert_array_equal(host(y32).view(np.uint32), y32_r.view(np.uint32))
        np.testing.assert_array_equal(host(y), y_r)
    assert ch.status() == 0


def test_chain_graph_replays():
    """A chain captured in a HIP graph: every replay, with new inputs copied
    in between, equals the oracle (and the eager run)."""
    announce("chain graph replays")
    M, dims = 5, (2048, 1024, 512)
    ch, outs, _ = _dependent_chain(M, dims, 1100)
    x_in = ch._steps[0].tensors[0]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ch.run()                               # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ch.run()
    for rep in range(4):
        bits = synth.activations_bf16(1110 + rep, M, dims[0], outliers=True)
        x_in.copy_(dev_bf16(bits))
        g.replay()
        torch.cuda.synchronize()
        ref, cur = [], bits
        for i in range(len(dims) - 1):
            (wq_r, ws_r), _ = _weights(1100 + 10 + i, dims[i + 1], dims[i])
            q_r, s_r = oracle.quantize_act(cur)
            _, y32_r, y_r = oracle.w8a8_linear(q_r, s_r, wq_r, ws_r)
            ref.append((q_r, s_r, y_r, y32_r))
            cur = y_r
        _check(outs, ref)
        ch.run()                               # eager run between replays
        torch.cuda.synchronize()
        _check(outs, ref)
    assert ch.status() == 0
