#!/usr/bin/env python3
"""Write tests/golden/lm_head_m5_1000.txt: the oracle's verdicts on the
LM-head verification workload (M = 5 rows = 4 drafts + 1, K = 4096,
V = 151936, int8 per-channel weights), 1000 trials.

Calls only the oracle and the seeded input generators:

* W ~ N(0, 0.02) fp32 [V][K] (synth.weights_f32, workload 3), quantized
  per output channel by the oracle;
* trial t: x = bf16(N(0,1)) [5][K] (synth.activations_bf16, workload 3,
  index t); the bf16 reference (the BF16 verifier's logits, fp64 sums of
  bf16 x times bf16 W) gives reference argmax ids a_ref[0..4]; the drafts
  copy a_ref's first p = t mod 5 ids and differ from a_ref at position p
  (synth.prefix_drafts);
* the oracle's W8A8 path gives argmax[0..4], accept_len and next_token.

The pages: verification with a quantized verifier, acceptance on the
dequantized logits, greedy decoding (gist.science Japanese summary,
技術的サマリー §2.2 items 3-4 and §4; gist.science Italian summary, Sommario
tecnico §2).  Run time about two minutes on 8 cores; memory about 20 GB.

    python tests/golden/make_lm_head_golden.py
"""
import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lm_head_m5_1000.txt")
TRIALS = 1000
G = 4
M = G + 1
K = 4096
V = synth.QWEN3_VOCAB
CHUNK = 250           # trials per fp64 product
NEAR_TIE = 1e-3       # top-2 gap of the fp32 logits below which a row is a near tie


def main():
    t0 = time.time()
    w = synth.weights_f32(synth.W_LM_HEAD, V, K)
    wq, ws = oracle.quantize_weight(w)
    print(f"weights quantized ({time.time() - t0:.0f} s)", flush=True)
    xs = [synth.activations_bf16(synth.W_LM_HEAD, M, K, index=t) for t in range(TRIALS)]

    a_ref = np.empty((TRIALS, M), dtype=np.int64)
    am = np.empty((TRIALS, M), dtype=np.int32)
    near = np.zeros((TRIALS, M), dtype=bool)
    gap_min = np.empty((TRIALS, M))
    for c0 in range(0, TRIALS, CHUNK):
        xb = np.concatenate(xs[c0:c0 + CHUNK])                  # [CHUNK*M][K] bf16 bits
        ref = oracle.bf16_reference_logits(xb, w)               # fp64
        a_ref[c0:c0 + CHUNK] = np.argmax(ref, axis=1).reshape(-1, M)
        del ref
        xq, xsc = oracle.quantize_act(xb)
        _, y32, _ = oracle.w8a8_linear(xq, xsc, wq, ws)
        am[c0:c0 + CHUNK] = oracle.argmax_rows(y32).reshape(-1, M)
        top2 = np.partition(y32, -2, axis=1)[:, -2:].astype(np.float64)
        gap = np.abs(top2[:, 1] - top2[:, 0]).reshape(-1, M)
        gap_min[c0:c0 + CHUNK] = gap
        near[c0:c0 + CHUNK] = gap < NEAR_TIE
        del y32
        print(f"trials {c0}..{c0 + CHUNK - 1} ({time.time() - t0:.0f} s)", flush=True)

    lines = []
    agree_prefix = 0
    for t in range(TRIALS):
        p = t % M
        d = synth.prefix_drafts(a_ref[t], p, V, synth.rng(synth.W_LM_HEAD, synth.T_DRAFT, t))
        al, nt = oracle.greedy_accept(d[None, :], am[t])
        if np.array_equal(am[t, :p + 1], a_ref[t, :p + 1]):
            agree_prefix += 1
            assert al[0] == p  # the accepted-length identity
        mask = int(sum(1 << i for i in range(M) if near[t, i]))
        lines.append(f"{t} {p} " + " ".join(map(str, d)) + " | " + " ".join(map(str, a_ref[t])) +
                     " | " + " ".join(map(str, am[t])) + f" | {al[0]} {nt[0]} | {mask}")
    flips = int(np.sum(am != a_ref))
    header = [
        "# Oracle verdicts for the LM-head verification workload: M=5 (4 drafts + 1),",
        "# K=4096, V=151936, int8 per-output-channel weights, 1000 trials.",
        "# Written by tests/golden/make_lm_head_golden.py (oracle + seeded synth inputs only).",
        "# Pages: a quantized verifier checks the drafted block; acceptance reads the",
        "# dequantized logits; greedy decoding (gist.science Japanese summary, 技術的サマリー",
        "# §2.2 items 3-4, §4; gist.science Italian summary, Sommario tecnico §2).",
        f"# w_scale_sha256: {hashlib.sha256(ws.tobytes()).hexdigest()}",
        f"# wq_sum: {int(wq.astype(np.int64).sum())}",
        f"# wq_row0_sha256: {hashlib.sha256(wq[0].tobytes()).hexdigest()}",
        f"# rows where the W8A8 argmax differs from the bf16 reference: {flips} of {TRIALS * M}",
        f"# trials whose W8A8 argmax agrees with the reference on rows 0..p: {agree_prefix}",
        f"# near-tie rows (top-2 fp32 logits within {NEAR_TIE}): {int(near.sum())}",
        "# columns: trial p drafts[4] | bf16-reference argmax[5] | W8A8 argmax[5] |",
        "#          accept_len next_token | near-tie row mask (bit i = row i)",
    ]
    with open(OUT, "w") as f:
        f.write("\n".join(header + lines) + "\n")
    print("\n".join(header[6:12]))
    print(f"wrote {OUT} ({time.time() - t0:.0f} s)")


if __name__ == "__main__":
    main()
