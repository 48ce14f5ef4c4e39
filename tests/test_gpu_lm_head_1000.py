"""The LM-head verification workload at full size on the GPU: M = 5 (4
drafts + 1), K = 4096, V = 151936, 1000 trials, against the oracle's
verdicts stored in tests/golden/lm_head_m5_1000.txt (written by
tests/golden/make_lm_head_golden.py from the oracle and the seeded inputs).

* the weights are drawn on the host from the same seeds, quantized on the
  GPU in the tiled layout: the per-channel scales must hash to the
  oracle's, the code sum must equal the oracle's, and sampled channels
  (un-tiled) must equal the oracle's codes for those channels;
* every trial runs quantize_act -> lm_head_verify with the stored drafts;
  argmax of all 5 rows, accept_len and next_token must equal the oracle's
  exactly (near-tie rows are reported, not excused).
"""
import hashlib
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import announce, dev, dev_bf16, gpu_available, host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lm_head_m5_1000.txt")
K, V, G = 4096, synth.QWEN3_VOCAB, 4
M = G + 1


def load_golden():
    meta, rows = {}, []
    for line in open(GOLDEN):
        if line.startswith("#"):
            if ":" in line:
                k, v = line[1:].split(":", 1)
                meta[k.strip()] = v.strip()
            continue
        head, ref, am, acc, mask = (p.split() for p in line.split("|"))
        rows.append({"t": int(head[0]), "p": int(head[1]),
                     "draft": np.array(head[2:], dtype=np.int32),
                     "a_ref": np.array(ref, dtype=np.int64), "am": np.array(am, dtype=np.int32),
                     "accept_len": int(acc[0]), "next_token": int(acc[1]), "near": int(mask[0])})
    return meta, rows


def untile(t: np.ndarray, N: int, Kk: int) -> np.ndarray:
    tiles, steps = t.shape[0], t.shape[1]
    a = t.reshape(tiles, steps, 4, 16, 16).transpose(0, 3, 1, 2, 4)
    return a.reshape(tiles * 16, steps * 64)[:N, :Kk]


@pytest.fixture(scope="module")
def lm_head():
    if not gpu_available():
        pytest.skip("no ROCm GPU")
    import w8a8_quantized_verification_amd as w8
    announce("LM head 151936 x 4096: draw weights on the host, quantize on the GPU")
    w = synth.weights_f32(synth.W_LM_HEAD, V, K)
    wd = dev(w)
    wt, ws = w8.quantize_weight(wd, tiled=True)
    torch.cuda.synchronize()
    del wd
    return w, wt, ws


def test_lm_head_weights_match_oracle(lm_head):
    import w8a8_quantized_verification_amd as w8  # noqa: F401
    w, wt, ws = lm_head
    meta, _ = load_golden()
    announce("LM head weight codes and scales")
    ws_h = host(ws)
    assert hashlib.sha256(ws_h.tobytes()).hexdigest() == meta["w_scale_sha256"]
    t = host(wt)
    assert int(t.astype(np.int64).sum()) == int(meta["wq_sum"])   # padding bytes are zero
    rows = np.concatenate([[0, 1, 15, 16, V - 1], np.random.default_rng(1).integers(0, V, 60)])
    full = untile(t, V, K)
    q_ref, s_ref = oracle.quantize_weight(synth.weight_rows_f32(synth.W_LM_HEAD, V, K, rows))
    np.testing.assert_array_equal(full[rows], q_ref)
    np.testing.assert_array_equal(ws_h[rows].view(np.uint32), s_ref.view(np.uint32))
    assert hashlib.sha256(full[0].tobytes()).hexdigest() == meta["wq_row0_sha256"]


def test_lm_head_1000_trials(lm_head):
    import w8a8_quantized_verification_amd as w8
    _, wt, ws = lm_head
    _, rows = load_golden()
    announce("LM head: 1000 verify trials")
    xs = np.concatenate([synth.activations_bf16(synth.W_LM_HEAD, M, K, index=t) for t in range(1000)])
    x_all = dev_bf16(xs)
    drafts = dev(np.stack([r["draft"] for r in rows]))
    am_all = torch.empty(1000, M, dtype=torch.int32, device="cuda:0")
    al_all = torch.empty(1000, dtype=torch.int32, device="cuda:0")
    nt_all = torch.empty(1000, dtype=torch.int32, device="cuda:0")
    xq = torch.empty(M, K, dtype=torch.int8, device="cuda:0")
    xsc = torch.empty(M, dtype=torch.float32, device="cuda:0")
    wsp = w8.Workspace()
    for t in range(1000):
        w8.quantize_act(x_all[t * M:(t + 1) * M], xq=xq, x_scale=xsc)
        w8.lm_head_verify(xq, xsc, wt, ws, drafts[t:t + 1], argmax=am_all[t],
                          accept_len=al_all[t:t + 1], next_token=nt_all[t:t + 1], workspace=wsp)
    torch.cuda.synchronize()
    am, al, nt = host(am_all), host(al_all), host(nt_all)
    want_am = np.stack([r["am"] for r in rows])
    want_al = np.array([r["accept_len"] for r in rows])
    want_nt = np.array([r["next_token"] for r in rows])
    near = sum(bin(r["near"]).count("1") for r in rows)
    known = sum(1 for r in rows if r["accept_len"] == r["p"])
    print(f"[gpu] near-tie rows: {near}; trials whose accepted length equals the built-in "
          f"prefix p: {known}/1000", flush=True)
    np.testing.assert_array_equal(am, want_am)
    np.testing.assert_array_equal(al, want_al)
    np.testing.assert_array_equal(nt, want_nt)
