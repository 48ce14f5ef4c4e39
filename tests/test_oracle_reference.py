"""Pins for the bf16 reference layer and the weight-traffic closed forms.

* the bf16 reference equals torch's CPU matmul of bf16-cast operands carried
  out in float64 (independent cast), and a float32 CPU matmul within the
  float32 summation bound K * 2^-23 * sum|x*w|;
* weight bytes: int8 + fp32 scales is N*K + 4N against bf16's 2*N*K, a ratio
  of 0.5 + 2/K (the halving of weight traffic);
* the latency model bytes/BW gives a BF16/INT8 time ratio that tends to 2.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import (bf16_linear_bytes, bf16_reference_logits, w8a8_linear_bytes,
                    weight_bytes_bf16, weight_bytes_int8)


def test_reference_against_torch_casts():
    M, N, K = 5, 300, 512
    x = synth.activations_bf16(81, M, K, outliers=True)
    w = synth.weights_f32(81, N, K)
    ref = bf16_reference_logits(x, w)
    xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    wt = torch.from_numpy(w).to(torch.bfloat16).to(torch.float64)
    t64 = (xt @ wt.T).numpy()
    np.testing.assert_allclose(ref, t64, rtol=0, atol=1e-12 * np.max(np.abs(t64)))
    t32 = (xt.float() @ wt.float().T).double().numpy()
    bound = K * 2.0 ** -23 * (xt.abs() @ wt.abs().T).numpy()
    assert np.all(np.abs(t32 - ref) <= bound)


@pytest.mark.parametrize("N,K", [(512, 256), (4096, 4096), (151936, 4096), (5120, 25600)])
def test_weight_bytes_halved(N, K):
    assert weight_bytes_bf16(N, K) == 2 * N * K
    assert weight_bytes_int8(N, K) == N * K + 4 * N
    assert weight_bytes_int8(N, K) / weight_bytes_bf16(N, K) == pytest.approx(0.5 + 2 / K)


def test_linear_bytes_examples():
    # LM head at M=5: 151936*4096 int8 + 4*151936 scales + 5*4096 + 20 + bf16 y + fp32 y
    b = w8a8_linear_bytes(5, 151936, 4096, y_bf16=True, y_f32=True)
    assert b == 151936 * 4096 + 4 * 151936 + 5 * 4096 + 4 * 5 + 2 * 5 * 151936 + 4 * 5 * 151936
    # the tiny verify linear (M=5, K=256, N=512) with its bf16 output
    assert w8a8_linear_bytes(5, 512, 256) == 139540
    # latency model: BF16 over INT8 time at equal bandwidth tends to 2 on large layers
    r = bf16_linear_bytes(5, 151936, 4096) / w8a8_linear_bytes(5, 151936, 4096)
    assert 1.99 < r < 2.0
