"""The allocation-free LM-head verification (w8a8_lm_head_verify_noalloc,
through the C ABI) against the workspace form (w8a8_lm_head_verify): two
calls in a row on the library's per-GPU scratch array — 288 verified rows
(32 sequences x 9, the batched kernel with the argmax fold), then 5 rows
(the skinny kernel) — must give bit-identical logits, argmax, accept_len
and next_token; a third call with more rows than the array holds is
rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import announce, dev, dev_bf16, gpu_available, host

pytestmark = pytest.mark.gpu

if gpu_available():
    import w8a8_quantized_verification_amd as w8
    from w8a8_quantized_verification_amd._lib import W8A8Error

W_NOALLOC = 41


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no ROCm GPU")


def _case(B, G, V, K, wt, ws, index):
    R = B * (G + 1)
    bits = synth.activations_bf16(W_NOALLOC, R, K, index=index)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    draft = synth.draft_ids(W_NOALLOC, B, G, V, index=index)
    return xq, xs, dev(draft)


def test_lm_head_verify_noalloc_matches_workspace_form():
    V, K = synth.QWEN3_VOCAB, 256
    w = synth.weights_f32(W_NOALLOC, V, K)
    wt, ws = w8.quantize_weight(dev(w), tiled=True)
    wsp = w8.Workspace()
    for call, (B, G) in enumerate([(32, 8), (1, 4)]):
        R = B * (G + 1)
        announce(f"lm_head_verify_noalloc call {call}: B={B} G={G} rows={R} V={V} K={K}")
        xq, xs, d = _case(B, G, V, K, wt, ws, call)
        # the drafts copy the first rows' argmax so that acceptance runs deep
        ref = w8.lm_head_verify(xq, xs, wt, ws, d, want_logits=True, workspace=wsp)
        torch.cuda.synchronize()
        am0 = host(ref[1]).reshape(B, G + 1)
        dd = host(d)
        for b in range(B):
            p = (b + call) % (G + 1)
            dd[b, :p] = am0[b, :p]
        d = dev(dd)
        ref = w8.lm_head_verify(xq, xs, wt, ws, d, want_logits=True, workspace=wsp)
        lg = torch.empty(R, V, dtype=torch.float32, device="cuda:0")
        am = torch.empty(R, dtype=torch.int32, device="cuda:0")
        al = torch.empty(B, dtype=torch.int32, device="cuda:0")
        nt = torch.empty(B, dtype=torch.int32, device="cuda:0")
        w8.lm_head_verify_noalloc(xq, xs, wt, ws, d, logits=lg, argmax=am, accept_len=al,
                                  next_token=nt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(lg).view(np.uint32), host(ref[0]).view(np.uint32))
        np.testing.assert_array_equal(host(am), host(ref[1]))
        np.testing.assert_array_equal(host(al), host(ref[2]))
        np.testing.assert_array_equal(host(nt), host(ref[3]))
        assert int(host(al).max()) > 0 or G == 0
    # more rows than the scratch array holds: rejected, nothing enqueued
    B, G = 33, 8
    announce(f"lm_head_verify_noalloc rejects B={B} G={G} ({B * (G + 1)} rows)")
    xq = torch.zeros(B * (G + 1), K, dtype=torch.int8, device="cuda:0")
    xs = torch.zeros(B * (G + 1), dtype=torch.float32, device="cuda:0")
    d = torch.zeros(B, G, dtype=torch.int32, device="cuda:0")
    with pytest.raises(W8A8Error, match="W8A8_NOALLOC_MAX_ROWS"):
        w8.lm_head_verify_noalloc(xq, xs, wt, ws, d)
