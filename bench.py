#!/usr/bin/env python3
"""Benchmark of the W8A8 verify hot path on one MI355X.

Headline workload: LM-head verification at M = 5 (4 drafts + 1) — hidden
4096, vocabulary 151936 (Qwen3-8B shapes), int8 per-channel weights, one
verify step = quantize_act -> w8a8_linear (fp32 logits) -> verify_accept
(argmax over the vocabulary + greedy acceptance of the 4 drafts).  It is the
only M = 5 workload that runs every step of the path.  Two copies of the
622 MB int8 LM head alternate between steps so that no step finds its
weights in the 256 MB Infinity Cache.

Printed: one JSON line with verified tokens/s (value), the roofline of the
dominant kernel (the LM-head GEMM: algorithmic bytes per launch over its
HIP-event-timed average duration, against 8 TB/s), the CPU oracle timed on
this host on a bounded sample, and secondary figures (per-linear GB/s of
the Qwen3-8B decoder-layer linears at M = 5 with weights rotated past the
cache, the in-build bf16 GEMM at the LM-head shape as the two-times-traffic
reference).

    python bench.py [--steps 200] [--warmup 20] [--no-cpu-baseline] [--no-extra]
    python bench.py --pmc-probe     # a short fixed run for rocprofv3 --pmc
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 verify GEMM HBM GB/s (% of peak) + verified tokens/s at M=5"
HBM_PEAK_GBS = 8000.0
PMC_FILE = os.path.join(ROOT, "profiles", "gemm_w8a8_lm_head_m5_traffic.txt")
GEMM_SRC = os.path.join(ROOT, "w8a8_quantized_verification_amd", "csrc", "gemm_w8a8.hip")


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-steps", type=int, default=3)
    p.add_argument("--no-extra", action="store_true")
    p.add_argument("--pmc-probe", action="store_true")
    return p.parse_args()


def lm_head_bytes(M, N, K):
    # int8 weight + fp32 scales + int8 activations + fp32 per-token scales + fp32 logits
    return N * K + 4 * N + M * K + 4 * M + 4 * M * N


def linear_bytes(M, N, K):
    # as above with the bf16 output a decoder-layer linear feeds onward
    return N * K + 4 * N + M * K + 4 * M + 2 * M * N


def file_sha(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per LM-head GEMM launch from the committed rocprofv3 --pmc
    summary, or None if absent or taken on a different kernel source."""
    if not os.path.exists(PMC_FILE):
        return None
    kv = {}
    for line in open(PMC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != file_sha(GEMM_SRC):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_int8_weight(N, K, seed, device):
    import torch
    import w8a8_quantized_verification_amd as w8
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32)
    w.mul_(0.02)
    wq, ws = w8.quantize_weight(w)
    wb = w.to(torch.bfloat16)
    del w
    return wq, ws, wb


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    M, K, V, G, B = 5, 4096, synth.QWEN3_VOCAB, 4, 1
    copies = [make_int8_weight(V, K, 1000 + i, dev) for i in range(2)]
    n_x = 8
    xs_host = [synth.activations_bf16(synth.W_LM_HEAD, M, K, index=i) for i in range(n_x)]
    x_dev = [torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(dev) for x in xs_host]
    draft = torch.from_numpy(synth.draft_ids(synth.W_LM_HEAD, B, G, V)).to(dev)
    xq = torch.empty(M, K, dtype=torch.int8, device=dev)
    xsc = torch.empty(M, dtype=torch.float32, device=dev)
    logits = torch.empty(M, V, dtype=torch.float32, device=dev)
    am = torch.empty(M, dtype=torch.int32, device=dev)
    al = torch.empty(B, dtype=torch.int32, device=dev)
    nt = torch.empty(B, dtype=torch.int32, device=dev)
    wsp = w8.Workspace()

    def step(i, ev=None):
        w8.quantize_act(x_dev[i % n_x], xq=xq, x_scale=xsc)
        wq, ws, _ = copies[i % 2]
        if ev is not None:
            ev[0].record()
        w8.linear(xq, xsc, wq, ws, want_bf16=False, y_f32=logits, workspace=wsp)
        if ev is not None:
            ev[1].record()
        w8.verify_accept(logits, draft, argmax=am, accept_len=al, next_token=nt, workspace=wsp)

    if args.pmc_probe:
        # fixed short run for counter collection: a plain 1 GiB copy (the
        # calibration kernel) then 8 LM-head steps
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        for i in range(8):
            step(i)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_probe": "done", "copy_bytes": 1 << 30,
                          "gemm_algorithmic_bytes": lm_head_bytes(M, V, K)}), flush=True)
        return

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(args.steps):
        step(i, evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    gemm_ms = [a.elapsed_time(b) for a, b in evs]
    gemm_avg_s = float(np.mean(gemm_ms)) / 1e3
    ms_per_step = total_ms / args.steps
    tok_s = M * args.steps / (total_ms / 1e3)
    bytes_launch = lm_head_bytes(M, V, K)
    achieved = bytes_launch / gemm_avg_s / 1e9
    traffic = read_traffic()

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,1) bf16 activations, N(0,0.02) weights quantized to int8 on the GPU)",
        "config": {"workload": "lm_head_verify_m5", "M": M, "K": K, "V": V, "B": B, "G": G,
                   "weights": "int8 per-output-channel, 2 rotating copies of 622 MB",
                   "step": "quantize_act + w8a8_linear(fp32 logits) + verify_accept"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "gemm_w8a8_skinny (LM head)",
                     "algorithmic_bytes_per_launch": bytes_launch,
                     "avg_launch_us": round(gemm_avg_s * 1e6, 3)},
        "gemm_gbs": round(achieved, 1),
        "gemm_frac_of_peak": round(achieved / HBM_PEAK_GBS, 4),
        "wall_s_timed": round(wall, 4),
    }

    if not args.no_extra:
        out["extra"] = extra_measurements(dev, copies, x_dev, xq, xsc, wsp)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(copies[0], xs_host, synth.draft_ids(synth.W_LM_HEAD, B, G, V),
                                           args.cpu_steps, M)
    print(json.dumps(out), flush=True)


def extra_measurements(dev, copies, x_dev, xq, xsc, wsp):
    """Secondary figures: Qwen3-8B decoder-layer linears at M=5 (8 rotating
    copies of the layer), and the bf16 reference GEMM at the LM-head shape."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    M = 5
    res = {}
    reps = 40
    nc = 8
    layer = []
    for li, lin in enumerate(synth.QWEN3_8B_LAYER):
        ws_list = [make_int8_weight(lin.N, lin.K, 2000 + 10 * li + c, dev)[:2] for c in range(nc)]
        x = torch.from_numpy(synth.activations_bf16(synth.W_LAYER_M5, M, lin.K, outliers=True)
                             .view(np.int16).copy()).view(torch.bfloat16).to(dev)
        lxq, lxs = w8.quantize_act(x)
        y = torch.empty(M, lin.N, dtype=torch.bfloat16, device=dev)
        for i in range(nc):
            w8.linear(lxq, lxs, *ws_list[i % nc], y_bf16=y, workspace=wsp)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda.synchronize()
        for i in range(reps):
            ev[i][0].record()
            w8.linear(lxq, lxs, *ws_list[i % nc], y_bf16=y, workspace=wsp)
            ev[i][1].record()
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(b) for a, b in ev])) / 1e3
        b = linear_bytes(M, lin.N, lin.K)
        layer.append({"name": lin.name, "N": lin.N, "K": lin.K, "us": round(t * 1e6, 2),
                      "GBs": round(b / t / 1e9, 1)})
        del ws_list
    tot_b = sum(linear_bytes(M, l.N, l.K) for l in synth.QWEN3_8B_LAYER)
    tot_t = sum(e["us"] for e in layer) / 1e6
    res["qwen3_8b_layer_linears_m5"] = {"per_linear": layer, "sum_us": round(tot_t * 1e6, 2),
                                        "aggregate_GBs": round(tot_b / tot_t / 1e9, 1),
                                        "aggregate_frac": round(tot_b / tot_t / 1e9 / HBM_PEAK_GBS, 4)}
    # bf16 reference at the LM-head shape (two-times weight traffic)
    K, V = 4096, synth.QWEN3_VOCAB
    xb = x_dev[0]
    yf = torch.empty(M, V, dtype=torch.float32, device=dev)
    for i in range(4):
        w8.bf16_linear(xb, copies[i % 2][2], want_bf16=False, y_f32=yf)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    torch.cuda.synchronize()
    for i in range(20):
        ev[i][0].record()
        w8.bf16_linear(xb, copies[i % 2][2], want_bf16=False, y_f32=yf)
        ev[i][1].record()
    torch.cuda.synchronize()
    tb = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    bb = 2 * V * K + 2 * M * K + 4 * M * V
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    lg = torch.empty(M, V, dtype=torch.float32, device=dev)
    for i in range(20):
        ev[i][0].record()
        w8.linear(xq, xsc, copies[i % 2][0], copies[i % 2][1], want_bf16=False, y_f32=lg, workspace=wsp)
        ev[i][1].record()
    torch.cuda.synchronize()
    ti = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    res["bf16_reference_lm_head_m5"] = {"us": round(tb * 1e6, 2), "GBs": round(bb / tb / 1e9, 1),
                                        "w8a8_us": round(ti * 1e6, 2),
                                        "time_ratio_bf16_over_w8a8": round(tb / ti, 3)}
    return res


def cpu_baseline(copy0, xs_host, draft, steps, M):
    """The oracle's verify step on this host's cores, on a bounded sample:
    ``steps`` LM-head steps with the same int8 weights (copied to the host)."""
    import numpy as np

    import oracle
    wq = copy0[0].cpu().numpy()
    ws = copy0[1].cpu().numpy()
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = os.cpu_count() or 1
    t0 = time.perf_counter()
    for i in range(steps):
        xq, xs = oracle.quantize_act(xs_host[i % len(xs_host)])
        _, y32, _ = oracle.w8a8_linear(xq, xs, wq, ws)
        oracle.verify_accept(y32, draft)
    dt = time.perf_counter() - t0
    return {"value": round(M * steps / dt, 3), "unit": "verified tokens/s", "cores": int(blas),
            "kind": "oracle",
            "sample": f"{steps} LM-head verify steps (M=5, K=4096, V=151936), numpy oracle, "
                      f"{dt:.1f} s; BLAS threads={blas}, elementwise steps single-threaded"}


if __name__ == "__main__":
    main()
