#!/usr/bin/env python3
"""Benchmark of the W8A8 verify hot path on one MI355X.

Headline workload: LM-head verification at M = 5 (4 drafts + 1) — hidden
4096, vocabulary 151936 (Qwen3-8B shapes), int8 per-output-channel weights
in the tiled layout.  One verify step = quantize_act -> lm_head_argmax (the
LM-head W8A8 linear with the row argmax folded into its epilogue) ->
accept_from_keys (greedy acceptance of the 4 drafts).  Two copies of the
622 MB int8 LM head alternate between steps so that no step finds its
weights in the 256 MB Infinity Cache.

Printed: one JSON line with verified tokens/s (value; eager launches, K
timed steps between synchronizations), the roofline of the dominant kernel
(the LM-head GEMM: algorithmic bytes per launch over its average duration from
HIP events that take the kernel's own start and end timestamps, against
8 TB/s; HBM traffic from the committed rocprofv3
counters), the CPU oracle timed on this host on a bounded sample, and
secondary figures ("extra"): the step as a HIP graph and through the
separate calls; the Qwen3-8B decoder-layer linears at M = 5 and M = 288
(TOPS and MFMA fraction); the row-major weight layout; the in-build bf16
GEMM at the LM-head shape (two-times-traffic reference); stochastic
verification at T = 1; the Qwen3-32B-shaped stack at M = 8 (int8 and bf16).

    python bench.py [--steps 200] [--warmup 20] [--no-cpu-baseline] [--no-extra]
                    [--no-stack]
    python bench.py --pmc-probe           # short fixed runs for rocprofv3 --pmc
    python bench.py --pmc-probe-batched
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
INT8_PEAK_TOPS = 5000.0   # dense int8 MFMA, MI355X
PMC_FILE = os.path.join(ROOT, "profiles", "gemm_w8a8_lm_head_m5_traffic.txt")
GEMM_SRC = os.path.join(ROOT, "w8a8_quantized_verification_amd", "csrc", "gemm_w8a8.hip")


TIMESTAMP_EVERY = 16   # timed steps per pair of kernel-timestamped ones


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-extra", action="store_true")
    p.add_argument("--no-stack", action="store_true",
                   help="skip the Qwen3-32B-shaped stack (96 GB of device memory)")
    p.add_argument("--pmc-probe", action="store_true")
    p.add_argument("--pmc-probe-batched", action="store_true",
                   help="short fixed run of the 288-row linears for rocprofv3 --pmc")
    p.add_argument("--ingest-pmc-batched", nargs="+", metavar="DIR",
                   help="rocprofv3 --pmc output dirs of --pmc-probe-batched runs")
    p.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn two rocprofv3 --pmc runs of --pmc-probe into the traffic summary")
    p.add_argument("--ingest-trace", metavar="TRACE_DIR",
                   help="turn a rocprofv3 --kernel-trace --stats csv run into a summary")
    p.add_argument("--command", default="", help="the command that produced the ingested run")
    p.add_argument("--stack32b-probe", action="store_true",
                   help="run STACK32B_LAYERS layers of the Qwen3-32B stack at M = 8 eagerly, "
                        "STACK32B_ROUNDS rounds, for rocprofv3 --kernel-trace")
    p.add_argument("--ingest-stack32b-trace", metavar="TRACE_DIR",
                   help="summarize a --stack32b-probe kernel trace into profiles/")
    p.add_argument("--layer288-probe", action="store_true",
                   help="only the fused 288-row Qwen3-8B layer linears, eager (for rocprofv3 "
                        "--kernel-trace)")
    p.add_argument("--ingest-layer288-trace", metavar="TRACE_DIR",
                   help="rocprofv3 --kernel-trace dir of a --layer288-probe run")
    p.add_argument("--batched-verify-probe", action="store_true",
                   help="only the 288-row LM-head verification step (for rocprofv3 --kernel-trace)")
    p.add_argument("--ingest-batched-trace", metavar="TRACE_DIR",
                   help="summary of a --kernel-trace --stats run of --batched-verify-probe")
    p.add_argument("--attention-probe", action="store_true",
                   help="only the attention scaling runs (for rocprofv3 --kernel-trace)")
    p.add_argument("--launch-probe", action="store_true",
                   help="only the launch-overhead runs (M=5 layer linears as a graph, the "
                        "headline step eager and as a graph) for rocprofv3 --kernel-trace")
    p.add_argument("--ingest-launch-trace", metavar="TRACE_DIR",
                   help="per-kernel duration and gap summary of a --kernel-trace run of "
                        "--launch-probe")
    p.add_argument("--ingest-attention-trace", metavar="TRACE_DIR",
                   help="per-launch-shape summary of a --kernel-trace run of --attention-probe")
    return p.parse_args()


def lm_head_bytes(M, N, K, logits=True):
    # int8 weight + fp32 scales + int8 activations + fp32 per-token scales
    # (+ fp32 logits when written)
    return N * K + 4 * N + M * K + 4 * M + (4 * M * N if logits else 0)


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


def read_batched_counters():
    """Per-shape MfmaUtil and HBM traffic over algorithmic bytes of the
    288-row kernels from the committed rocprofv3 --pmc summary, with
    ``stale`` set when the summary was taken on another source of the
    batched kernels than the one built here."""
    path = os.path.join(ROOT, "profiles", "gemm_w8a8_batched_m288_counters.txt")
    src = os.path.join(ROOT, "w8a8_quantized_verification_amd", "csrc", "gemm_w8a8_batched.hip")
    if not os.path.exists(path):
        return None
    out, cur, sha = {}, None, None
    for line in open(path):
        line = line.rstrip()
        if line.startswith("[") and "]" in line:
            cur = line[1:line.index("]")]
            out[cur] = {}
        elif line.startswith("kernel_source_sha:"):
            sha = line.split(":", 1)[1].strip()
        elif cur and ":" in line and not line.startswith("#"):
            k, v = (x.strip() for x in line.split(":", 1))
            if k in ("MfmaUtil", "hbm_over_algorithmic", "duration_us_under_counters"):
                out[cur][k] = float(v)
    return {"per_shape": out, "kernel_source_sha": sha, "stale": sha != file_sha(src),
            "source": "profiles/gemm_w8a8_batched_m288_counters.txt"}


def make_weight(N, K, workload, index, device, tiled=True, with_bf16=False):
    """Random-init N(0, 0.02) fp32 weight drawn on the device (seeded by
    workload and index), quantized to int8 per output channel by the library;
    optionally also its bf16 copy, row-major (with_bf16=True) or in the tiled
    bf16 layout (with_bf16="tiled")."""
    import torch
    import synth
    import w8a8_quantized_verification_amd as w8
    w = synth.weights_device(workload, index, N, K, device)
    wq, ws = w8.quantize_weight(w, tiled=tiled)
    wb = w.to(torch.bfloat16) if with_bf16 else None
    del w
    if with_bf16 == "tiled":
        wb = w8.tile_weight_bf16(wb)
    return wq, ws, wb


def graph_time(fns, replays=20, execs=2):
    """Capture the callables into ``execs`` identical HIP graphs and replay
    them in turn; return the mean time of one replay in seconds (a replay
    runs every callable once, in order).  Alternating two graph execs keeps
    the stream fed: replaying one exec back to back leaves a ~9 us bubble at
    every replay boundary (kernel trace of --launch-probe)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gs = []
    for _ in range(execs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        gs.append(g)
    for i in range(3 * execs):
        gs[i % execs].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(replays):
        gs[i % execs].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / replays / 1e3


def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        rows.extend(csv.DictReader(open(f)))
    return rows


GEMM_KERNEL = "gemm_w8a8_skinny<2, 4, 10, true, true>"
COPY_KERNEL_HINT = "copy"


def ingest_pmc(fetch_dir, write_dir, command):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the LM-head GEMM, each
    scaled by what the same counter reads for the 1 GiB copy of the probe."""
    import numpy as np
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _csv_rows(d, "counter_collection.csv") if r["Counter_Name"] == name]
        gemm = [float(r["Counter_Value"]) for r in rows if GEMM_KERNEL in r["Kernel_Name"]]
        copy = [float(r["Counter_Value"]) for r in rows
                if COPY_KERNEL_HINT in r["Kernel_Name"].lower() and GEMM_KERNEL not in r["Kernel_Name"]]
        if not gemm or not copy:
            raise SystemExit(f"{name}: no GEMM or copy dispatch found in {d}")
        kib_copy = max(copy)          # the 1 GiB copy: its largest dispatch
        factor = (1 << 30) / (kib_copy * 1024.0)
        kib = float(np.median(gemm))
        out[name] = (kib, kib_copy, factor, kib * 1024.0 * factor)
    M, K, V = 5, 4096, 151936
    alg = lm_head_bytes(M, V, K, logits=False) + 8 * M * ((V + 31) // 32)
    total = out["FETCH_SIZE"][3] + out["WRITE_SIZE"][3]
    lines = [
        "# HBM traffic of the LM-head W8A8 GEMM (M=5, K=4096, V=151936, tiled int8, fused argmax)",
        f"# kernel: {GEMM_KERNEL}",
        f"# commands: {command}",
        "# counters are KiB per dispatch (median over the probe's 8 GEMM dispatches); each is",
        "# scaled by (2^30 bytes) / (the same counter on the probe's 1 GiB copy dispatch)",
    ]
    for name, (kib, kib_copy, factor, b) in out.items():
        lines.append(f"{name.lower()}_kib_per_dispatch: {kib:.1f}")
        lines.append(f"{name.lower()}_copy_kib: {kib_copy:.1f}")
        lines.append(f"{name.lower()}_scale: {factor:.5f}")
        lines.append(f"{name.lower()}_bytes_per_launch: {b:.0f}")
    lines += [f"hbm_bytes_per_launch: {total:.0f}",
              f"algorithmic_bytes_per_launch: {alg}",
              f"traffic_over_algorithmic: {total / alg:.4f}",
              f"kernel_source_sha: {file_sha(GEMM_SRC)}"]
    os.makedirs(os.path.dirname(PMC_FILE), exist_ok=True)
    with open(PMC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def ingest_trace(trace_dir, command, out_path):
    """Short text summary of a rocprofv3 --kernel-trace --stats csv run: per
    kernel the average, median, minimum and maximum duration and the call
    count (the median from the per-dispatch kernel trace)."""
    import numpy as np
    rows = _csv_rows(trace_dir, "kernel_stats.csv")
    per = {}
    for r in _csv_rows(trace_dir, "kernel_trace.csv"):
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# rocprofv3 kernel statistics", f"# command: {command}",
             f"{'avg_us':>10} {'median_us':>10} {'min_us':>10} {'max_us':>10} {'calls':>6}  kernel"]
    for r in rows:
        n = r["Name"]
        med = float(np.median(per[n])) if n in per else float("nan")
        if len(n) > 110:
            n = n[:107] + "..."
        lines.append(f"{float(r['AverageNs']) / 1e3:10.2f} {med:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {int(r['Calls']):6d}  {n}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


ATTENTION_WORKLOADS = [(1, 5, 32, 8, 4096), (1, 8, 64, 8, 4096), (1, 5, 32, 8, 16384),
                       (1, 8, 64, 8, 65536), (1, 5, 32, 8, 65536), (32, 5, 32, 8, 4096)]


def ingest_attention_trace(trace_dir, command, out_path):
    """Median durations of the split and combine kernels per workload of a
    rocprofv3 --kernel-trace csv run of --attention-probe.  Each split
    launch is paired with the combine launch after it; the workloads run in
    ATTENTION_WORKLOADS order, and adjacent ones differ in their (split
    kernel, split grid, combine grid), which is where a new one starts."""
    import numpy as np
    rows = sorted((r for r in _csv_rows(trace_dir, "kernel_trace.csv") if "attn_" in r["Kernel_Name"]),
                  key=lambda r: int(r["Start_Timestamp"]))

    def grid(r):
        return f"{r['Grid_Size_X']}x{r['Grid_Size_Y']}x{r['Grid_Size_Z']}"

    segs, sig = [], None
    for a, b in zip(rows, rows[1:]):
        if "split" not in a["Kernel_Name"] or "combine" not in b["Kernel_Name"]:
            continue
        s_ = (a["Kernel_Name"].split("(")[0].replace("void ", ""), grid(a), grid(b))
        if s_ != sig:
            segs.append((s_, [], []))
            sig = s_
        segs[-1][1].append(int(a["End_Timestamp"]) - int(a["Start_Timestamp"]))
        segs[-1][2].append(int(b["End_Timestamp"]) - int(b["Start_Timestamp"]))
    lines = ["# rocprofv3 kernel trace of verify_attention (the attention_scaling workloads)",
             f"# command: {command}",
             "# medians over the calls of each workload; grid = work-items x, y, z",
             f"{'split_us':>9} {'combine_us':>10} {'calls':>6}  {'split kernel':<32} "
             f"{'split grid':<12} workload (B, T, Hq, Hkv, positions)"]
    for k, ((name, g1, g2), sp, cb) in enumerate(segs):
        wl = ATTENTION_WORKLOADS[k] if k < len(ATTENTION_WORKLOADS) else "?"
        lines.append(f"{np.median(sp) / 1e3:9.2f} {np.median(cb) / 1e3:10.2f} {len(sp):6d}  "
                     f"{name:<32} {g1:<12} {wl}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


BATCHED_SHAPES = ("q", "gate", "down")   # probe order; 4 dispatches each
BATCHED_PMC_FILE = os.path.join(ROOT, "profiles", "gemm_w8a8_batched_m288_counters.txt")
BATCHED_SRC = os.path.join(ROOT, "w8a8_quantized_verification_amd", "csrc", "gemm_w8a8_batched.hip")


def pmc_probe_batched(dev):
    """A plain 1 GiB copy (the traffic calibration), then 4 launches of each
    288-row Qwen3-8B linear in BATCHED_SHAPES, alternating 2 weight copies."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    del src, dst
    M = 288
    for name in BATCHED_SHAPES:
        lin = next(l for l in synth.QWEN3_8B_LAYER if l.name == name)
        wl = [make_weight(lin.N, lin.K, synth.W_BATCHED, 7000 + c, dev)[:2] for c in range(2)]
        x = torch.from_numpy(synth.activations_bf16(synth.W_BATCHED, M, lin.K, outliers=True)
                             .view(np.int16).copy()).view(torch.bfloat16).to(dev)
        xq, xs = w8.quantize_act(x)
        y = torch.empty(M, lin.N, dtype=torch.bfloat16, device=dev)
        for i in range(4):
            w8.linear(xq, xs, *wl[i % 2], y_bf16=y)
        xt, xts = w8.quantize_act_tiled(x)
        for i in range(4):
            w8.linear_tiled_act(xt, xts, *wl[i % 2], K=lin.K, y_bf16=y)
        torch.cuda.synchronize()
        del wl
    print(json.dumps({"pmc_probe_batched": "done", "shapes": BATCHED_SHAPES}), flush=True)


def split_of(kernel_name):
    """The k split (KS, the last template argument) of a gemm_w8a8_lds32
    kernel name, else 1."""
    import re
    m = re.search(r"gemm_w8a8_lds32<([^>]*)>", kernel_name)
    return int(m.group(1).split(",")[-1]) if m else 1


def ingest_pmc_batched(dirs, command):
    """Per-shape medians of the counters found in the --pmc-probe-batched runs:
    HBM bytes (FETCH_SIZE/WRITE_SIZE, scaled by the 1 GiB copy as for the
    LM-head GEMM) against the algorithmic bytes, and MfmaUtil (rocprofv3's
    derived MFMA-busy percentage) beside the utilisation implied by the
    kernel durations."""
    import numpy as np

    import synth
    M = 288
    # both activation layouts run the register-fragment kernel or one of the
    # LDS-pipelined ones, by shape; the probe's dispatch order tells them apart
    batched_kernel = lambda k: "gemm_w8a8_batched" in k or "gemm_w8a8_lds" in k  # noqa: E731
    variants = (("row_major_act", batched_kernel), ("tiled_act", batched_kernel))
    per = {(n, v): {} for n in BATCHED_SHAPES for v, _ in variants}
    kname = {}
    for d in dirs:
        rows = _csv_rows(d, "counter_collection.csv")
        for cname in sorted({r["Counter_Name"] for r in rows}):
            rr = [r for r in rows if r["Counter_Name"] == cname]
            scale = 1.0
            if cname in ("FETCH_SIZE", "WRITE_SIZE"):
                copy = [float(r["Counter_Value"]) for r in rr if "copy" in r["Kernel_Name"].lower()]
                scale = (1 << 30) / (max(copy) * 1024.0) * 1024.0   # KiB -> calibrated bytes
            # the probe: per shape, 4 row-major-activation launches then 4 tiled ones
            gem = sorted([r for r in rr if "gemm_w8a8_batched" in r["Kernel_Name"]
                          or "gemm_w8a8_lds" in r["Kernel_Name"]],
                         key=lambda r: int(r["Dispatch_Id"]))
            if len(gem) != 8 * len(BATCHED_SHAPES):
                raise SystemExit(f"{d}: {cname}: expected {8 * len(BATCHED_SHAPES)} batched "
                                 f"dispatches, found {len(gem)}")
            for i, n in enumerate(BATCHED_SHAPES):
                for j, (v, tag) in enumerate(variants):
                    sel = gem[8 * i + 4 * j:8 * i + 4 * j + 4]
                    if not all(tag(r["Kernel_Name"]) for r in sel):
                        raise SystemExit(f"{d}: unexpected kernel order for {n} {v}")
                    kname[(n, v)] = sel[0]["Kernel_Name"].split("(w8a8")[0].replace("void ", "")
                    vals = [float(r["Counter_Value"]) * scale for r in sel]
                    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
                            for r in sel]
                    per[(n, v)][cname] = float(np.median(vals))
                    per[(n, v)].setdefault("dur_s", []).extend(durs)
    lines = ["# Counters of the batched W8A8 GEMM at M=288 (Qwen3-8B linears, tiled int8 weights),",
             "# with row-major activations (w8a8_linear_tiled) and tiled activations",
             "# (w8a8_linear_tiled_act)",
             *[f"# kernel ({n}, {v}): {k[:110]}" for (n, v), k in kname.items()],
             f"# commands: {command}",
             "# per shape: medians over 4 dispatches.  FETCH_SIZE/WRITE_SIZE in bytes, calibrated",
             "# by the probe's 1 GiB copy.  MfmaUtil = 100*sum(SQ_VALU_MFMA_BUSY_CYCLES) /",
             "# (max(GRBM_GUI_ACTIVE)*SIMD_NUM).  implied_mfma_pct = 2*M*N*K / duration / 5.0 POPS,",
             "# with the duration taken from the same dispatches under the counter run.",
             "# model_activations_once_per_xcd = (algorithmic + 7*M*K) / algorithmic: the traffic",
             "# if each of the 8 XCDs (separate L2s) fetches the activations once and the",
             "# weights are fetched once; for a kernel that splits k across KS workgroups",
             "# (last template argument) model_with_split_handoff adds the handoff: each slice",
             "# writes its int32 partial, the last arriver reads the KS-1 others and zeroes all",
             "# KS (per wave 96 x 32 int32 per slice, 4 waves per 96 x 128 tile)"]
    for n in BATCHED_SHAPES:
        lin = next(l for l in synth.QWEN3_8B_LAYER if l.name == n)
        alg = linear_bytes(M, lin.N, lin.K)
        for v, _ in variants:
            e = per[(n, v)]
            dur = float(np.median(e.pop("dur_s")))
            lines.append(f"[{n} {v}] N={lin.N} K={lin.K}")
            lines.append(f"  duration_us_under_counters: {dur * 1e6:.2f}")
            lines.append(f"  implied_mfma_pct: {100 * 2 * M * lin.N * lin.K / dur / 5.0e15:.2f}")
            for k, val in sorted(e.items()):
                lines.append(f"  {k}: {val:.1f}")
            if "FETCH_SIZE" in e and "WRITE_SIZE" in e:
                lines.append(f"  algorithmic_bytes: {alg}")
                lines.append(f"  hbm_over_algorithmic: {(e['FETCH_SIZE'] + e['WRITE_SIZE']) / alg:.3f}")
                # each of the 8 XCDs fetches the M x K activations into its own L2
                lines.append(f"  model_activations_once_per_xcd: {(alg + 7 * M * lin.K) / alg:.3f}")
                ks = split_of(kname[(n, v)])
                if ks > 1:
                    slot = 96 * 32 * 4   # bytes of one wave's partial
                    slots = -(-lin.N // 128) * -(-M // 96) * 4
                    handoff = slots * slot * (ks + (ks - 1) + ks)
                    lines.append(f"  split_handoff_bytes: {handoff}")
                    lines.append(f"  model_with_split_handoff: "
                                 f"{(alg + 7 * M * lin.K + handoff) / alg:.3f}")
    lines.append(f"kernel_source_sha: {file_sha(BATCHED_SRC)}")
    with open(BATCHED_PMC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.command)
        return
    if args.ingest_pmc_batched:
        ingest_pmc_batched(args.ingest_pmc_batched, args.command)
        return
    if args.ingest_trace:
        ingest_trace(args.ingest_trace, args.command,
                     os.path.join(ROOT, "profiles", "lm_head_verify_m5_kernel_trace.txt"))
        return
    if args.ingest_layer288_trace:
        ingest_layer288_trace(args.ingest_layer288_trace, args.command,
                              os.path.join(ROOT, "profiles", "batched_layer_m288_kernel_trace.txt"))
        return
    if args.ingest_stack32b_trace:
        ingest_stack32b_trace(args.ingest_stack32b_trace, args.command,
                              os.path.join(ROOT, "profiles", "stack32b_m8_kernel_trace.txt"))
        return
    if args.ingest_batched_trace:
        ingest_trace(args.ingest_batched_trace, args.command,
                     os.path.join(ROOT, "profiles", "lm_head_verify_m288_kernel_trace.txt"))
        return
    if args.ingest_launch_trace:
        ingest_launch_trace(args.ingest_launch_trace, args.command,
                            os.path.join(ROOT, "profiles", "launch_gaps_m5_kernel_trace.txt"))
        return
    if args.ingest_attention_trace:
        ingest_attention_trace(args.ingest_attention_trace, args.command,
                               os.path.join(ROOT, "profiles", "verify_attention_kernel_trace.txt"))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    if args.attention_probe:
        print(json.dumps({"attention_scaling": attention_scaling(torch.device("cuda:0"))}),
              flush=True)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.layer288_probe:
        layer288_probe(dev)
        return
    if args.stack32b_probe:
        stack32b_probe(dev)
        return

    M, K, V, G, B = 5, 4096, synth.QWEN3_VOCAB, 4, 1
    # The LM head of the 1000-trial verification workload: fp32 N(0, 0.02)
    # drawn on the host from the workload's seeds, quantized to int8 by the
    # library.  A second copy of the same codes at another address
    # alternates with it, so no step finds its weights in the 256 MB
    # Infinity Cache (and both give the same verdicts).
    wall_setup = time.perf_counter()
    w_host = synth.weights_f32(synth.W_LM_HEAD, V, K)
    w_dev = torch.from_numpy(w_host).to(dev)
    wq0, ws0 = w8.quantize_weight(w_dev, tiled=True)
    del w_dev
    copies = [(wq0, ws0, None), (wq0.clone(), ws0, None)]
    torch.cuda.synchronize()
    print(f"[bench] LM head drawn and quantized ({time.perf_counter() - wall_setup:.1f} s)",
          file=sys.stderr, flush=True)
    if args.batched_verify_probe:
        print(json.dumps({"batched_verify_step_m288":
                          batched_verify_measurement(dev, copies, w8.Workspace())}), flush=True)
        return
    # the 1000 trials: hidden rows x_t and drafts whose first p = t mod 5
    # ids copy the bf16-reference argmax (stored with the oracle's verdicts)
    trials = read_lm_head_trials()
    n_trials = len(trials["draft"])
    xs_host = [synth.activations_bf16(synth.W_LM_HEAD, M, K, index=t) for t in range(n_trials)]
    x_all = torch.from_numpy(np.concatenate(xs_host).view(np.int16).copy()).view(
        torch.bfloat16).to(dev)
    x_dev = [x_all[t * M:(t + 1) * M] for t in range(n_trials)]
    drafts = torch.from_numpy(trials["draft"]).to(dev)
    n_slots = max(args.steps, 2) + 128
    am_all = torch.empty(n_slots, M, dtype=torch.int32, device=dev)
    al_all = torch.empty(n_slots, dtype=torch.int32, device=dev)
    nt_all = torch.empty(n_slots, dtype=torch.int32, device=dev)
    xq = torch.empty(M, K, dtype=torch.int8, device=dev)
    xsc = torch.empty(M, dtype=torch.float32, device=dev)
    logits = torch.empty(M, V, dtype=torch.float32, device=dev)
    am, al, nt = am_all[0], al_all[0:1], nt_all[0:1]
    draft = drafts[0:1]
    wsp = w8.Workspace()

    def step(i, ev=None, slot=None):
        """One verify step of trial i mod 1000: quantize its 5 hidden rows,
        then the LM-head linear with the argmax's first pass fused into its
        epilogue, then greedy acceptance of its 4 drafts (the logits
        themselves are not written); the verdict goes to result slot
        ``slot`` (default i).  With ``ev``, the LM-head kernel records its
        own start and end timestamps into the two events (no marker packets
        join the stream)."""
        t = i % n_trials
        j = i if slot is None else slot
        w8.quantize_act(x_dev[t], xq=xq, x_scale=xsc)
        wq, ws, _ = copies[i % 2]
        w8.lm_head_argmax(xq, xsc, wq, ws, workspace=wsp, events=ev)
        w8.accept_from_keys(drafts[t:t + 1], argmax=am_all[j], accept_len=al_all[j:j + 1],
                            next_token=nt_all[j:j + 1], workspace=wsp)

    def step_separate(i):
        """The same step through the three separate calls, fp32 logits written."""
        t = i % n_trials
        w8.quantize_act(x_dev[t], xq=xq, x_scale=xsc)
        wq, ws, _ = copies[i % 2]
        w8.linear(xq, xsc, wq, ws, want_bf16=False, y_f32=logits, workspace=wsp)
        w8.verify_accept(logits, drafts[t:t + 1], argmax=am, accept_len=al, next_token=nt,
                         workspace=wsp)

    if args.pmc_probe_batched:
        pmc_probe_batched(dev)
        return
    if args.launch_probe:
        launch_probe(dev, step, wsp)
        return
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
                          "gemm_algorithmic_bytes": lm_head_bytes(M, V, K, logits=False)
                          + 8 * M * ((V + 31) // 32)}), flush=True)
        return

    for i in range(args.warmup):
        step(i, slot=n_slots - 1)
    torch.cuda.synchronize()
    # The LM-head kernel's own timestamps are taken on two consecutive steps
    # (both weight copies) of every 16: a timestamped launch costs the eager
    # step ~7 us (100.2 -> 107.6 us per step, measured back to back), so
    # timing every launch would understate the step rate.
    sampled = [(i // 2) % (TIMESTAMP_EVERY // 2) == 0 for i in range(args.steps)]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           if s else None for s in sampled]
    for e in evs:               # torch creates each event on its first record
        if e is not None:
            e[0].record()
            e[1].record()
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
    gemm_ms = [e[0].elapsed_time(e[1]) for e in evs if e is not None]
    gemm_avg_s = float(np.mean(gemm_ms)) / 1e3
    ms_per_step = total_ms / args.steps
    tok_s = M * args.steps / (total_ms / 1e3)
    # the verdicts of the timed steps against the oracle's (stored per trial)
    t_idx = np.arange(args.steps) % n_trials
    al_h = al_all[:args.steps].cpu().numpy()
    nt_h = nt_all[:args.steps].cpu().numpy()
    am_h = am_all[:args.steps].cpu().numpy()
    verdicts_ok = int(np.sum((al_h == trials["accept_len"][t_idx])
                             & (nt_h == trials["next_token"][t_idx])
                             & np.all(am_h == trials["argmax"][t_idx], axis=1)))
    emitted = int(np.sum(al_h + 1))
    emitted_tok_s = emitted / (total_ms / 1e3)
    # gemm_ms: the LM-head kernel's own durations on the sampled steps (its
    # start and end timestamps, recorded into the events by hipExtLaunchKernel)
    # the fused kernel reads the weights, scales and activations; its only
    # writes are the atomic folds of the row maxima (8 bytes per row per
    # 32-channel workgroup)
    bytes_launch = lm_head_bytes(M, V, K, logits=False) + 8 * M * ((V + 31) // 32)
    achieved = bytes_launch / gemm_avg_s / 1e9
    traffic = read_traffic()
    # after the timed region: 128 steps with every LM-head launch
    # timestamped (distribution of the kernel's duration), then the
    # streaming-read probe over the same weight bytes (the read bandwidth a
    # plain stream sustains here)
    lat = kernel_timestamp_run(step, n_slots - 128, 128)
    probe = hbm_probe_run(w8, [c[0] for c in copies], 32)
    achievable = probe["mean_GBs"]

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
        "data": "synthetic (seeded N(0,1) bf16 activations; N(0,0.02) fp32 weights drawn on the "
                "host, quantized to int8 by the library; drafts copy a prefix of p = t mod 5 "
                "bf16-reference argmax ids per trial t)",
        "config": {"workload": "lm_head_verify_m5", "M": M, "K": K, "V": V, "B": B, "G": G,
                   "trials": n_trials,
                   "weights": "int8 per-output-channel, tiled layout, 2 rotating copies of 622 MB",
                   "step": "quantize_act + lm_head_argmax (LM-head W8A8 linear with the "
                           "argmax folded into its epilogue) + accept_from_keys (greedy "
                           "acceptance)",
                   "launch": "eager, one stream",
                   "kernel_timestamps": f"2 of every {TIMESTAMP_EVERY} steps"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "gemm_w8a8_skinny<2,4,10,tiled,argmax> (LM head 4096->151936, M=5)",
                     "algorithmic_bytes_per_launch": bytes_launch,
                     "avg_launch_us": round(gemm_avg_s * 1e6, 3),
                     "launches_timed": len(gemm_ms),
                     "achievable": round(achievable, 1),
                     "frac_of_achievable": round(achieved / achievable, 4),
                     "achievable_probe": probe,
                     "kernel_timestamps_128": lat,
                     "median_launch_us": lat["median_us"],
                     "achieved_at_median": round(bytes_launch / (lat["median_us"] * 1e-6) / 1e9, 1)},
        "emitted_tokens_per_s": round(emitted_tok_s, 1),
        "mean_tokens_emitted_per_step": round(emitted / args.steps, 4),
        "verdicts_match_oracle": f"{verdicts_ok}/{args.steps}",
        "gemm_gbs": round(achieved, 1),
        "gemm_frac_of_peak": round(achieved / HBM_PEAK_GBS, 4),
        "wall_s_timed": round(wall, 4),
    }

    if not args.no_extra:
        extra = {}
        # the whole step as one HIP graph (two steps per graph: both weight copies)
        t_graph = graph_time([lambda: step(0), lambda: step(1)], replays=50) / 2
        extra["graph_step"] = {"ms_per_step": round(t_graph * 1e3, 5),
                               "verified_tokens_per_s": round(M / t_graph, 1)}
        t_sep = graph_time([lambda: step_separate(0), lambda: step_separate(1)], replays=50) / 2
        extra["graph_step_separate_calls"] = {"ms_per_step": round(t_sep * 1e3, 5),
                                              "verified_tokens_per_s": round(M / t_sep, 1)}
        extra.update(extra_measurements(dev, copies, x_dev, xq, xsc, wsp))
        extra["gemm_w8a8_batched_m288_counters"] = read_batched_counters()
        if not args.no_stack:
            extra["qwen3_32b_stack_m8"] = stack32b_measurement(dev, wsp)
        out["extra"] = extra

    if not args.no_cpu_baseline and not args.no_extra:
        out["extra"]["oracle_timings"] = oracle_timings()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w_host, xs_host, trials["draft"], args.cpu_seconds, M)
    print(json.dumps(out), flush=True)


GOLDEN = os.path.join(ROOT, "tests", "golden", "lm_head_m5_1000.txt")


def read_lm_head_trials(path=GOLDEN):
    """The 1000-trial LM-head workload's drafts and the oracle's verdicts
    (written by tests/golden/make_lm_head_golden.py from the oracle and the
    seeded inputs): per trial t, p = t mod 5, drafts[4], argmax[5],
    accept_len, next_token."""
    import numpy as np
    drafts, am, al, nt, p = [], [], [], [], []
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        head, _ref, a, acc, _mask = (x.split() for x in line.split("|"))
        p.append(int(head[1]))
        drafts.append([int(v) for v in head[2:]])
        am.append([int(v) for v in a])
        al.append(int(acc[0]))
        nt.append(int(acc[1]))
    return {"draft": np.array(drafts, dtype=np.int32), "argmax": np.array(am, dtype=np.int32),
            "accept_len": np.array(al, dtype=np.int32), "next_token": np.array(nt, dtype=np.int32),
            "p": np.array(p, dtype=np.int32)}


def kernel_timestamp_run(step, slot0, n):
    """``n`` verify steps with every LM-head launch timestamped (its own
    start and end, see ``lm_head_argmax(events=)``): mean, median, p10 and
    p90 of the kernel's duration."""
    import numpy as np
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for e in evs:
        e[0].record()
        e[1].record()
    torch.cuda.synchronize()
    for i in range(n):
        step(i, evs[i], slot=slot0 + i)
    torch.cuda.synchronize()
    us = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
    return {"launches": n, "mean_us": round(float(us.mean()), 3),
            "median_us": round(float(np.median(us)), 3),
            "p10_us": round(float(np.percentile(us, 10)), 3),
            "p90_us": round(float(np.percentile(us, 90)), 3),
            "min_us": round(float(us.min()), 3)}


def hbm_probe_run(w8, bufs, n):
    """The library's streaming-read probe over the given buffers (the LM
    head's weight copies, alternating): ``n`` launches, each timed by its
    own kernel timestamps; GB/s = bytes / duration."""
    import numpy as np
    import torch
    nbytes = bufs[0].numel() * bufs[0].element_size()
    sink = torch.empty(w8.HBM_PROBE_SINK_WORDS, dtype=torch.int32, device=bufs[0].device)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for e in evs:
        e[0].record()
        e[1].record()
    for i in range(2):
        w8.hbm_read_probe(bufs[i % len(bufs)], sink=sink)
    torch.cuda.synchronize()
    for i in range(n):
        w8.hbm_read_probe(bufs[i % len(bufs)], sink=sink, events=evs[i])
    torch.cuda.synchronize()
    us = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bytes": int(nbytes), "launches": n, "mean_us": round(float(us.mean()), 3),
            "median_us": round(float(np.median(us)), 3),
            "mean_GBs": round(float(nbytes / (us.mean() * 1e-6) / 1e9), 1),
            "best_GBs": round(float(gbs.max()), 1),
            "kernel": "hbm_read_kernel (16-byte non-temporal loads, one contiguous 32 KiB chunk per 256-thread workgroup)"}


LAUNCH_PHASES = ("layer linears M=5 (graph: qkv, o, gate_up, down; 2 weight sets)",
                 "headline step, eager (quantize_act, lm_head_argmax, accept_from_keys)",
                 "headline step, one HIP graph exec of 2 steps replayed",
                 "headline step, two HIP graph execs of 2 steps replayed in turn")


def launch_probe(dev, step, wsp, reps=20):
    """Three phases separated by 50 ms of idle time, for a kernel trace:
    the Qwen3-8B layer's fused linears at M = 5 replayed as one HIP graph
    (two weight sets, so 8 launches per replay), ``reps`` eager headline
    steps, and ``reps`` headline steps replayed as a graph of two."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8
    M = 5
    lins = synth.QWEN3_8B_LAYER
    groups = ((0, 1, 2), (3,), (4, 5), (6,))
    sets = []
    for c in range(2):
        row = []
        for gi, grp in enumerate(groups):
            N, K = sum(lins[i].N for i in grp), lins[grp[0]].K
            w = torch.cat([synth.weights_device(synth.W_LAYER_M5, 9000 + 100 * gi + 10 * c + i,
                                                lins[i].N, K, dev) for i in grp])
            wq, ws = w8.quantize_weight(w, tiled=True)
            del w
            x = torch.from_numpy(synth.activations_bf16(synth.W_LAYER_M5, M, K, outliers=True)
                                 .view(np.int16).copy()).view(torch.bfloat16).to(dev)
            xq, xs = w8.quantize_act(x)
            row.append((xq, xs, wq, ws, torch.empty(M, N, dtype=torch.bfloat16, device=dev)))
        sets.append(row)
    lw = w8.Workspace()
    fns = [(lambda a=a: w8.linear(a[0], a[1], a[2], a[3], y_bf16=a[4], workspace=lw))
           for row in sets for a in row]
    torch.cuda.synchronize()
    time.sleep(0.05)
    graph_time(fns, replays=reps)
    torch.cuda.synchronize()
    time.sleep(0.05)
    for i in range(reps):
        step(i)
    torch.cuda.synchronize()
    time.sleep(0.05)
    graph_time([lambda: step(0), lambda: step(1)], replays=reps // 2, execs=1)
    torch.cuda.synchronize()
    time.sleep(0.05)
    graph_time([lambda: step(0), lambda: step(1)], replays=reps // 2, execs=2)
    torch.cuda.synchronize()
    print(json.dumps({"launch_probe": "done", "phases": LAUNCH_PHASES}), flush=True)


def ingest_launch_trace(trace_dir, command, out_path):
    """Per-phase summary of a --kernel-trace run of --launch-probe: for each
    kernel (name and grid), the median duration and the median gap between
    the end of the kernel before it and its start; phases are told apart by
    idle time over 10 ms, warm-up launches (graph capture, first replays)
    are dropped by taking the last replays only."""
    import numpy as np
    rows = _csv_rows(trace_dir, "kernel_trace.csv")
    ev = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"],
                  int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)) for r in rows))
    phases, cur = [], []
    for e in ev:
        if cur and e[0] - cur[-1][1] > 10_000_000:
            phases.append(cur)
            cur = []
        cur.append(e)
    if cur:
        phases.append(cur)
    phases = phases[-len(LAUNCH_PHASES):]
    lines = ["# Kernel durations and launch gaps: rocprofv3 --kernel-trace of bench.py --launch-probe",
             f"# command: {command}",
             "# gap = start of a kernel minus end of the kernel before it (same stream)",
             "# per kernel (name, grid threads): median duration, median gap before it, count"]
    for title, ph in zip(LAUNCH_PHASES, phases):
        half = ph[len(ph) // 2:]             # the later half: past capture and warm-up
        stats = {}
        for k in range(1, len(half)):
            s0, e0, name, grid = half[k]
            key = (name.split("(")[0].replace("void ", ""), grid)
            stats.setdefault(key, {"dur": [], "gap": []})
            stats[key]["dur"].append((e0 - s0) / 1e3)
            stats[key]["gap"].append((s0 - half[k - 1][1]) / 1e3)
        span = (half[-1][1] - half[0][0]) / 1e3
        lines.append(f"[{title}] kernels {len(half)}, span {span:.1f} us")
        for (name, grid), v in stats.items():
            n = name if len(name) <= 70 else name[:67] + "..."
            lines.append(f"  {np.median(v['dur']):9.2f} us dur  {np.median(v['gap']):7.2f} us gap "
                         f"{len(v['dur']):5d}  grid {grid:9d}  {n}")
    lines += launch_breakdown(phases[0][len(phases[0]) // 2:], phases[1])
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def launch_breakdown(layer, headline):
    """Per-launch split of the M = 5 layer phase of --launch-probe (graph
    replays cycling qkv, o, gate_up, down, the widest grid being gate_up)
    into the gap before the launch, a fixed per-launch cost (ramp to full
    streaming plus the tail) and the streaming of its bytes: a least-squares
    line duration = c + bytes / R through the four launches and the
    headline LM-head GEMM (eager phase) gives c and R."""
    import numpy as np

    import synth
    M = 5
    lins = synth.QWEN3_8B_LAYER
    shapes = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))
    big = max(e[3] for e in layer)
    per = {n: {"dur": [], "gap": []} for n, _ in shapes}
    for j in range(3, len(layer) - 1):
        if layer[j][3] != big:
            continue
        for off, (n, _) in zip((-2, -1, 0, 1), shapes):
            s0, e0 = layer[j + off][0], layer[j + off][1]
            per[n]["dur"].append((e0 - s0) / 1e3)
            per[n]["gap"].append((s0 - layer[j + off - 1][1]) / 1e3)
    head = [(e[1] - e[0]) / 1e3 for e in headline if "skinny" in e[2]]
    rows = []
    for n, grp in shapes:
        N, K = sum(lins[i].N for i in grp), lins[grp[0]].K
        rows.append((n, linear_bytes(M, N, K), float(np.median(per[n]["dur"])),
                     float(np.median(per[n]["gap"])), len(per[n]["dur"]), float(np.max(per[n]["gap"]))))
    lm = synth.QWEN3_8B_LM_HEAD
    hb = linear_bytes(M, lm.N, lm.K)
    pts_b = [r[1] for r in rows] + ([hb] if head else [])
    pts_d = [r[2] for r in rows] + ([float(np.median(head))] if head else [])
    slope, c = np.polyfit(np.array(pts_b, float), np.array(pts_d, float), 1)
    rate = 1.0 / slope / 1e6   # TB/s (bytes per us -> TB/s)
    out = ["[layer linears M=5: per launch, duration = fixed + bytes / R]",
           f"  least squares over the four launches and the headline LM head "
           f"({hb / 1e6:.1f} MB, {np.median(head) if head else float('nan'):.2f} us): "
           f"fixed c = {c:.2f} us per launch, R = {rate:.2f} TB/s",
           "  (medians over the replays; gap = idle time before the launch, its maximum marks the",
           "  boundaries between graph replays)",
           f"  {'launch':8s} {'MB':>8s} {'dur_us':>8s} {'gap_us':>7s} {'gap_max':>7s} {'fixed_us':>8s} "
           f"{'stream_us':>9s} {'resid_us':>8s} {'n':>4s}"]
    tot = {"dur": 0.0, "gap": 0.0, "stream": 0.0}
    for n, b, d, g, cnt, gmax in rows:
        st = b * slope
        out.append(f"  {n:8s} {b / 1e6:8.2f} {d:8.2f} {g:7.2f} {gmax:7.2f} {c:8.2f} {st:9.2f} "
                   f"{d - c - st:8.2f} {cnt:4d}")
        tot["dur"] += d
        tot["gap"] += g
        tot["stream"] += st
    out.append(f"  layer: {tot['dur']:.2f} us in the four launches + {tot['gap']:.2f} us of gaps; "
               f"{4 * c:.2f} us of it fixed per-launch cost, {tot['stream']:.2f} us streaming at R")
    return out


def rotation_copies(N, K):
    """Distinct weight copies a graph cycles through so that the weights of
    one pass (>= 600 MB) cannot sit in the 256 MB Infinity Cache."""
    return int(min(128, max(8, -(-600_000_000 // (N * K)))))


def layer_measurement(dev, wsp, M, workload):
    """The Qwen3-8B decoder-layer linears at M rows: each linear graph-replayed
    over enough distinct weight copies to defeat the Infinity Cache; GB/s of
    the algorithmic bytes and int8 TOPS (2*M*N*K) against the 5.0 POPS dense
    int8 MFMA peak."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    layer = []
    for li, lin in enumerate(synth.QWEN3_8B_LAYER):
        nc = rotation_copies(lin.N, lin.K)
        wl = [make_weight(lin.N, lin.K, workload, 2000 + 200 * li + c, dev)[:2] for c in range(nc)]
        x = torch.from_numpy(synth.activations_bf16(workload, M, lin.K, outliers=True)
                             .view(np.int16).copy()).view(torch.bfloat16).to(dev)
        lxq, lxs = w8.quantize_act(x)
        y = torch.empty(M, lin.N, dtype=torch.bfloat16, device=dev)
        fns = [(lambda c=c: w8.linear(lxq, lxs, *wl[c], y_bf16=y, workspace=wsp)) for c in range(nc)]
        t = graph_time(fns, replays=10) / nc
        b = linear_bytes(M, lin.N, lin.K)
        tops = 2 * M * lin.N * lin.K / t / 1e12
        e = {"name": lin.name, "N": lin.N, "K": lin.K, "copies": nc,
             "us": round(t * 1e6, 2), "GBs": round(b / t / 1e9, 1),
             "TOPS": round(tops, 1), "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)}
        if M <= 16:
            # the in-build bf16 GEMM at the same shape (twice the weight bytes),
            # over its own rotating bf16 copies in the tiled bf16 layout
            ncb = rotation_copies(lin.N, 2 * lin.K)
            wb = [w8.tile_weight_bf16(synth.weights_device(workload, 2000 + 200 * li + c, lin.N,
                                                           lin.K, dev).to(torch.bfloat16))
                  for c in range(ncb)]
            yb16 = torch.empty(M, lin.N, dtype=torch.bfloat16, device=dev)
            tb = graph_time([(lambda c=c: w8.bf16_linear(x, wb[c], N=lin.N, y_bf16=yb16))
                             for c in range(ncb)], replays=10) / ncb
            e.update({"bf16_us": round(tb * 1e6, 2),
                      "bf16_GBs": round((2 * lin.N * lin.K + 2 * M * lin.K + 2 * M * lin.N)
                                        / tb / 1e9, 1),
                      "time_ratio_bf16_over_w8a8": round(tb / t, 3)})
            del wb
        if M > 16:
            # the same product with the activations quantized into the tiled layout
            xt, xts = w8.quantize_act_tiled(x)
            fns = [(lambda c=c: w8.linear_tiled_act(xt, xts, *wl[c], K=lin.K, y_bf16=y))
                   for c in range(nc)]
            tt = graph_time(fns, replays=10) / nc
            tt_tops = 2 * M * lin.N * lin.K / tt / 1e12
            e.update({"tiled_act_us": round(tt * 1e6, 2), "tiled_act_TOPS": round(tt_tops, 1),
                      "tiled_act_mfma_frac": round(tt_tops / INT8_PEAK_TOPS, 4)})
        layer.append(e)
        del wl
    tot_b = sum(linear_bytes(M, l.N, l.K) for l in synth.QWEN3_8B_LAYER)
    tot_ops = sum(2 * M * l.N * l.K for l in synth.QWEN3_8B_LAYER)
    tot_t = sum(e["us"] for e in layer) / 1e6
    extra = {}
    if M <= 16:
        tb = sum(e["bf16_us"] for e in layer) / 1e6
        extra = {"bf16_sum_us": round(tb * 1e6, 2),
                 "time_ratio_bf16_over_w8a8": round(tb / tot_t, 3)}
    if M > 16:
        tt = sum(e["tiled_act_us"] for e in layer) / 1e6
        extra = {"tiled_act_sum_us": round(tt * 1e6, 2),
                 "tiled_act_aggregate_TOPS": round(tot_ops / tt / 1e12, 1),
                 "tiled_act_aggregate_mfma_frac": round(tot_ops / tt / 1e12 / INT8_PEAK_TOPS, 4)}
    return {"M": M, "per_linear": layer, "sum_us": round(tot_t * 1e6, 2), **extra,
            "aggregate_GBs": round(tot_b / tot_t / 1e9, 1),
            "aggregate_frac": round(tot_b / tot_t / 1e9 / HBM_PEAK_GBS, 4),
            "aggregate_TOPS": round(tot_ops / tot_t / 1e12, 1),
            "aggregate_mfma_frac": round(tot_ops / tot_t / 1e12 / INT8_PEAK_TOPS, 4),
            "timing": "HIP graph over the rotating weight copies, mean of 10 replays"}


def batched_verify_measurement(dev, copies, wsp):
    """Batched verification: 32 sequences x (8 drafts + 1) = 288 rows
    through the LM head (4096 -> 151936) with greedy acceptance, two
    alternating 622 MB LM-head copies, as a HIP graph.  Tiled activations
    (quantize_act_tiled -> lm_head_argmax_tiled_act -> accept_from_keys)
    against row-major ones (quantize_act -> lm_head_argmax ->
    accept_from_keys)."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    B, G, K, V = 32, 8, 4096, synth.QWEN3_VOCAB
    M = B * (G + 1)
    xs_l = [torch.from_numpy(synth.activations_bf16(synth.W_BATCHED, M, K, index=i)
                             .view(np.int16).copy()).view(torch.bfloat16).to(dev) for i in range(2)]
    draft = torch.from_numpy(synth.draft_ids(synth.W_BATCHED, B, G, V)).to(dev)
    xt = torch.empty(w8.tiled_shape(M, K), dtype=torch.int8, device=dev)
    xq = torch.empty(M, K, dtype=torch.int8, device=dev)
    xsc = torch.empty(M, dtype=torch.float32, device=dev)
    am = torch.empty(M, dtype=torch.int32, device=dev)
    al = torch.empty(B, dtype=torch.int32, device=dev)
    nt = torch.empty(B, dtype=torch.int32, device=dev)

    def step_tiled(i):
        w8.quantize_act_tiled(xs_l[i % 2], xq_tiled=xt, x_scale=xsc)
        w8.lm_head_argmax_tiled_act(xt, xsc, copies[i % 2][0], copies[i % 2][1], K=K,
                                    workspace=wsp)
        w8.accept_from_keys(draft, argmax=am, accept_len=al, next_token=nt, workspace=wsp)

    def step_rows(i):
        w8.quantize_act(xs_l[i % 2], xq=xq, x_scale=xsc)
        w8.lm_head_argmax(xq, xsc, copies[i % 2][0], copies[i % 2][1], workspace=wsp)
        w8.accept_from_keys(draft, argmax=am, accept_len=al, next_token=nt, workspace=wsp)

    t_t = graph_time([lambda: step_tiled(0), lambda: step_tiled(1)], replays=10) / 2
    t_r = graph_time([lambda: step_rows(0), lambda: step_rows(1)], replays=5) / 2
    ops = 2 * M * V * K
    return {"B": B, "G": G, "M": M, "ms_per_step": round(t_t * 1e3, 4),
            "verified_tokens_per_s": round(M / t_t, 1),
            "lm_head_TOPS": round(ops / t_t / 1e12, 1),
            "lm_head_mfma_frac": round(ops / t_t / 1e12 / INT8_PEAK_TOPS, 4),
            "row_major_ms_per_step": round(t_r * 1e3, 4),
            "step": "quantize_act_tiled + lm_head_argmax_tiled_act + accept_from_keys",
            "timing": "HIP graph, 2 LM-head copies alternating"}


def w4a8_measurement(dev, x_dev, xq, xsc, wsp):
    """The W4A8 verifier (int4 per-channel weights): the LM-head verify step
    at M = 5 (quantize_act -> lm_head_argmax_w4 -> accept_from_keys) with
    two alternating 311 MB int4 copies of the LM head, the fused GEMM's
    weight-read rate, and the Qwen3-8B layer linears at M = 5 in int4."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    M, K, V, G, B = 5, 4096, synth.QWEN3_VOCAB, 4, 1

    def w4(N, Kk, workload, index):
        w = synth.weights_device(workload, index, N, Kk, dev)
        out = w8.quantize_weight_w4(w)
        del w
        return out

    cp = [w4(V, K, synth.W_LM_HEAD, 1000 + i) for i in range(2)]
    draft = torch.from_numpy(synth.draft_ids(synth.W_LM_HEAD, B, G, V)).to(dev)
    am = torch.empty(M, dtype=torch.int32, device=dev)
    al = torch.empty(B, dtype=torch.int32, device=dev)
    nt = torch.empty(B, dtype=torch.int32, device=dev)

    def step(i):
        w8.quantize_act(x_dev[i % len(x_dev)], xq=xq, x_scale=xsc)
        w8.lm_head_argmax_w4(xq, xsc, *cp[i % 2], workspace=wsp)
        w8.accept_from_keys(draft, argmax=am, accept_len=al, next_token=nt, workspace=wsp)

    t_step = graph_time([lambda: step(0), lambda: step(1)], replays=50) / 2
    t_gemm = graph_time([lambda: w8.lm_head_argmax_w4(xq, xsc, *cp[0], workspace=wsp),
                         lambda: w8.accept_from_keys(draft, argmax=am, accept_len=al,
                                                     next_token=nt, workspace=wsp),
                         lambda: w8.lm_head_argmax_w4(xq, xsc, *cp[1], workspace=wsp),
                         lambda: w8.accept_from_keys(draft, argmax=am, accept_len=al,
                                                     next_token=nt, workspace=wsp)],
                        replays=50) / 2
    wbytes = V * K // 2 + 4 * V + M * K + 4 * M + 8 * M * ((V + 31) // 32)
    res = {"ms_per_step": round(t_step * 1e3, 5), "verified_tokens_per_s": round(M / t_step, 1),
           "lm_head_plus_accept_us": round(t_gemm * 1e6, 2),
           "lm_head_weight_GBs_incl_accept": round(wbytes / t_gemm / 1e9, 1),
           "int4_weight_bytes": V * K // 2,
           "timing": "HIP graph; 2 int4 LM-head copies alternating"}
    del cp
    layer = []
    for li, lin in enumerate(synth.QWEN3_8B_LAYER):
        nc = rotation_copies(lin.N, lin.K // 2)
        wl = [w4(lin.N, lin.K, synth.W_LAYER_M5, 3000 + 200 * li + c) for c in range(nc)]
        x = torch.from_numpy(synth.activations_bf16(synth.W_LAYER_M5, M, lin.K, outliers=True)
                             .view(np.int16).copy()).view(torch.bfloat16).to(dev)
        lxq, lxs = w8.quantize_act(x)
        y = torch.empty(M, lin.N, dtype=torch.bfloat16, device=dev)
        t = graph_time([(lambda c=c: w8.linear_w4(lxq, lxs, *wl[c], y_bf16=y)) for c in range(nc)],
                       replays=10) / nc
        b = lin.N * lin.K // 2 + 4 * lin.N + M * lin.K + 4 * M + 2 * M * lin.N
        layer.append({"name": lin.name, "us": round(t * 1e6, 2), "GBs": round(b / t / 1e9, 1)})
        del wl
    res["qwen3_8b_layer_linears_m5"] = {"per_linear": layer,
                                        "sum_us": round(sum(e["us"] for e in layer), 2)}
    return res


LAYER288_GROUPS = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))
LAYER288_ROUNDS = 12


def layer288_probe(dev):
    """The fused 288-row layer's four launches (tiled activations, bf16 out,
    the layer's workspace), eager, LAYER288_ROUNDS rounds over rotating weight
    copies, in the order of LAYER288_GROUPS (for rocprofv3 --kernel-trace)."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    M = 288
    lins = synth.QWEN3_8B_LAYER
    wsp = w8.Workspace()
    shapes = []
    for gi, (name, grp) in enumerate(LAYER288_GROUPS):
        N, K = sum(lins[i].N for i in grp), lins[grp[0]].K
        nc = rotation_copies(N, K)
        wl = []
        for c in range(nc):
            w = torch.cat([synth.weights_device(synth.W_LAYER_M5, 7000 + 100 * gi + 10 * c + i,
                                                lins[i].N, K, dev) for i in grp])
            wl.append(w8.quantize_weight(w, tiled=True))
            del w
        x = torch.from_numpy(synth.activations_bf16(synth.W_LAYER_M5, M, K, outliers=True)
                             .view(np.int16).copy()).view(torch.bfloat16).to(dev)
        xt, xs = w8.quantize_act_tiled(x)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        shapes.append((wl, xt, xs, y, K))
    torch.cuda.synchronize()
    for r in range(LAYER288_ROUNDS):
        for wl, xt, xs, y, K in shapes:
            w8.linear_tiled_act(xt, xs, *wl[r % len(wl)], K=K, y_bf16=y, workspace=wsp)
    torch.cuda.synchronize()
    print(json.dumps({"layer288_probe": "done", "rounds": LAYER288_ROUNDS}), flush=True)


def ingest_layer288_trace(trace_dir, command, out_path):
    """Per-shape durations of the --layer288-probe launches: the batched
    kernels' dispatches in start order are the rounds of (qkv, o, gate_up,
    down); the first round is left out (first touch of the code and data)."""
    import numpy as np

    import synth
    rows = sorted((r for r in _csv_rows(trace_dir, "kernel_trace.csv")
                   if "gemm_w8a8_lds" in r["Kernel_Name"] or "gemm_w8a8_batched" in r["Kernel_Name"]),
                  key=lambda r: int(r["Start_Timestamp"]))
    n = len(LAYER288_GROUPS)
    if len(rows) != n * LAYER288_ROUNDS:
        raise SystemExit(f"expected {n * LAYER288_ROUNDS} batched dispatches, found {len(rows)}")
    lins = synth.QWEN3_8B_LAYER
    lines = ["# rocprofv3 kernel trace of the fused 288-row Qwen3-8B layer (tiled activations,",
             "# bf16 outputs, weights rotated past the Infinity Cache), one eager launch per shape",
             f"# and round, rounds 2..{LAYER288_ROUNDS}", f"# command: {command}",
             f"{'shape':>8} {'N':>6} {'K':>6} {'avg_us':>8} {'median_us':>9} {'min_us':>8} "
             f"{'max_us':>8} {'TOPS@med':>9} {'wgs':>5}  kernel"]
    tot, ops_all = 0.0, 0
    for gi, (name, grp) in enumerate(LAYER288_GROUPS):
        N, K = sum(lins[i].N for i in grp), lins[grp[0]].K
        sel = rows[n + gi::n]
        d = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel])
        med = float(np.median(d))
        ops = 2 * 288 * N * K
        wgs = int(sel[0]["Grid_Size_X"]) // max(int(sel[0]["Workgroup_Size_X"]), 1)
        kname = sel[0]["Kernel_Name"].split("(w8a8")[0].replace("void ", "")
        lines.append(f"{name:>8} {N:6d} {K:6d} {d.mean():8.2f} {med:9.2f} {d.min():8.2f} "
                     f"{d.max():8.2f} {ops / med / 1e6:9.1f} {wgs:5d}  {kname}")
        tot += med
        ops_all += ops
    lines.append(f"layer (sum of medians): {tot:.2f} us, {ops_all / tot / 1e6:.1f} TOPS "
                 f"({ops_all / tot / 1e6 / INT8_PEAK_TOPS:.4f} of the int8 MFMA peak)")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


STACK32B_LAYERS = 8     # 4 GB of int8 weights: past the 256 MB Infinity Cache
STACK32B_ROUNDS = 6
STACK32B_GROUPS = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))


def stack32b_probe(dev):
    """STACK32B_LAYERS layers of the Qwen3-32B stack at M = 8 as the stack
    measurement runs them (per layer and fused group: quantize_act of the
    group's input, then the linear; weights drawn on the device), eager,
    STACK32B_ROUNDS rounds, for rocprofv3 --kernel-trace."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    M = 8
    lins = synth.QWEN3_32B_LAYER
    wsp = w8.Workspace()
    layers = []
    for layer in range(STACK32B_LAYERS):
        row = []
        for j, (name, grp) in enumerate(STACK32B_GROUPS):
            K = lins[grp[0]].K
            w = torch.cat([synth.weights_device(synth.W_STACK32B,
                                                synth.stack_tensor_index(layer, li),
                                                lins[li].N, K, dev) for li in grp])
            wq, ws = w8.quantize_weight(w, tiled=True)
            del w
            b = synth.activations_bf16(synth.W_STACK32B, M, K, index=10_000 + 4 * layer + j,
                                       outliers=True, layer=layer)
            x = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(dev)
            y = torch.empty(M, ws.shape[0], dtype=torch.bfloat16, device=dev)
            row.append((x, wq, ws, y))
        layers.append(row)
    xq = {k: torch.empty(M, k, dtype=torch.int8, device=dev)
          for k in {lins[g[0]].K for _, g in STACK32B_GROUPS}}
    xsc = torch.empty(M, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for r in range(STACK32B_ROUNDS):
        for row in layers:
            for (x, wq, ws, y) in row:
                k = x.shape[1]
                w8.quantize_act(x, xq=xq[k], x_scale=xsc)
                w8.linear(xq[k], xsc, wq, ws, y_bf16=y, workspace=wsp)
    torch.cuda.synchronize()
    print(json.dumps({"stack32b_probe": "done", "layers": STACK32B_LAYERS,
                      "rounds": STACK32B_ROUNDS}), flush=True)


def ingest_stack32b_trace(trace_dir, command, out_path):
    """Per-launch durations of the --stack32b-probe: in start order the
    rounds of (per layer, per fused group: quantize_act, linear); the first
    round is left out (first touch of the code and data)."""
    import numpy as np

    import synth
    rows = sorted((r for r in _csv_rows(trace_dir, "kernel_trace.csv")
                   if "quantize_rows_kernel" in r["Kernel_Name"]
                   or "gemm_w8a8_skinny" in r["Kernel_Name"]),
                  key=lambda r: int(r["Start_Timestamp"]))
    n = STACK32B_LAYERS * len(STACK32B_GROUPS) * 2
    if len(rows) < n * STACK32B_ROUNDS:
        raise SystemExit(f"expected {n * STACK32B_ROUNDS} dispatches, found {len(rows)}")
    rows = rows[-n * STACK32B_ROUNDS:]   # the rounds follow the weights' own quantization
    lins = synth.QWEN3_32B_LAYER
    lines = ["# rocprofv3 kernel trace of the Qwen3-32B linear stack at M = 8 (tiled int8 weights,",
             f"# bf16 outputs), {STACK32B_LAYERS} layers x {STACK32B_ROUNDS} eager rounds "
             f"(rounds 2..{STACK32B_ROUNDS} kept; {STACK32B_LAYERS} layers = 4 GB, past the",
             "# Infinity Cache); per fused group its quantize_act launch and its linear",
             f"# command: {command}",
             f"{'launch':>18} {'N':>6} {'K':>6} {'median_us':>9} {'min_us':>8} {'max_us':>8} "
             f"{'TB/s@med':>8} {'grid_wgs':>8}  kernel"]
    per_layer = 0.0
    for j, (name, grp) in enumerate(STACK32B_GROUPS):
        N, K = sum(lins[i].N for i in grp), lins[grp[0]].K
        for part in (0, 1):
            sel = [rows[rd * n + layer * len(STACK32B_GROUPS) * 2 + 2 * j + part]
                   for rd in range(1, STACK32B_ROUNDS) for layer in range(STACK32B_LAYERS)]
            d = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel])
            med = float(np.median(d))
            wgs = int(sel[0]["Grid_Size_X"]) * int(sel[0].get("Grid_Size_Y", 1) or 1) // \
                max(int(sel[0]["Workgroup_Size_X"]), 1)
            kname = sel[0]["Kernel_Name"].split("(w8a8")[0].split("(")[0].replace("void ", "")
            label = f"{name} {'quantize' if part == 0 else 'linear'}"
            tbs = "" if part == 0 else f"{(N * K + 4 * N + 8 * K + 2 * 8 * N) / med / 1e6:8.2f}"
            lines.append(f"{label:>18} {N if part else 0:6d} {K:6d} {med:9.2f} {d.min():8.2f} "
                         f"{d.max():8.2f} {tbs:>8} {wgs:8d}  {kname}")
            per_layer += med
    lines.append(f"per layer (sum of medians): {per_layer:.2f} us; x 64 layers = "
                 f"{per_layer * 64 / 1e3:.3f} ms of kernel time before the LM head")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def fused_layer_measurement(dev, wsp, M, tiled_act=False):
    """The Qwen3-8B layer's linears at M rows with q/k/v and gate/up fused
    (their output channels stacked in one weight, per-channel codes and
    scales unchanged): 4 launches instead of 7, each graph-replayed over
    enough weight copies to pass 600 MB.  With ``tiled_act`` the
    activations go in the tiled layout (the batched kernels' fast path)."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    lins = synth.QWEN3_8B_LAYER
    groups = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))
    out, tot_t, tot_b = [], 0.0, 0
    for gi, (name, grp) in enumerate(groups):
        N, K = sum(lins[i].N for i in grp), lins[grp[0]].K
        nc = rotation_copies(N, K)
        wl = []
        for c in range(nc):
            w = torch.cat([synth.weights_device(synth.W_LAYER_M5, 7000 + 100 * gi + 10 * c + i,
                                                lins[i].N, K, dev) for i in grp])
            wl.append(w8.quantize_weight(w, tiled=True))
            del w
        x = torch.from_numpy(synth.activations_bf16(synth.W_LAYER_M5, M, K, outliers=True)
                             .view(np.int16).copy()).view(torch.bfloat16).to(dev)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        if tiled_act:
            lxq, lxs = w8.quantize_act_tiled(x)
            t = graph_time([(lambda c=c: w8.linear_tiled_act(lxq, lxs, *wl[c], K=K, y_bf16=y))
                            for c in range(nc)], replays=10) / nc
        else:
            lxq, lxs = w8.quantize_act(x)
            t = graph_time([(lambda c=c: w8.linear(lxq, lxs, *wl[c], y_bf16=y, workspace=wsp))
                            for c in range(nc)], replays=10) / nc
        b = linear_bytes(M, N, K)
        e = {"name": name, "N": N, "K": K, "copies": nc, "us": round(t * 1e6, 2),
             "GBs": round(b / t / 1e9, 1)}
        if M > 16:
            e["TOPS"] = round(2 * M * N * K / t / 1e12, 1)
            e["mfma_frac"] = round(2 * M * N * K / t / 1e12 / INT8_PEAK_TOPS, 4)
        out.append(e)
        tot_t += t
        tot_b += b
        del wl
    res = {"M": M, "per_launch": out, "sum_us": round(tot_t * 1e6, 2),
           "aggregate_GBs": round(tot_b / tot_t / 1e9, 1),
           "aggregate_frac": round(tot_b / tot_t / 1e9 / HBM_PEAK_GBS, 4),
           "timing": "HIP graph over the rotating weight copies, mean of 10 replays"}
    if M > 16:
        ops = 2 * M * sum(l.N * l.K for l in lins)
        res["aggregate_TOPS"] = round(ops / tot_t / 1e12, 1)
        res["aggregate_mfma_frac"] = round(ops / tot_t / 1e12 / INT8_PEAK_TOPS, 4)
        res["activations"] = "tiled" if tiled_act else "row-major"
    return res


def extra_measurements(dev, copies, x_dev, xq, xsc, wsp):
    """Secondary figures: Qwen3-8B decoder-layer linears at M=5 (8 rotating
    copies of each weight, graph-replayed), the row-major layout and the
    bf16 reference GEMM at the LM-head shape."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    M = 5
    res = {}
    res["qwen3_8b_layer_linears_m5"] = layer_measurement(dev, wsp, M, synth.W_LAYER_M5)
    res["qwen3_8b_layer_linears_m5_fused"] = fused_layer_measurement(dev, wsp, M)
    res["qwen3_8b_layer_linears_m288"] = layer_measurement(dev, wsp, 288, synth.W_BATCHED)
    res["qwen3_8b_layer_linears_m288_fused"] = fused_layer_measurement(dev, wsp, 288,
                                                                       tiled_act=True)
    res["library_gemm_reference"] = library_int8_gemm(dev)

    K, V = 4096, synth.QWEN3_VOCAB
    lg = torch.empty(M, V, dtype=torch.float32, device=dev)

    def ev_time(fn, reps=20):
        for i in range(4):
            fn(i)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda.synchronize()
        for i in range(reps):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3

    # row-major weight layout at the LM-head shape
    rm = [make_weight(V, K, synth.W_LM_HEAD, 1000 + i, dev, tiled=False, with_bf16=True)
          for i in range(2)]
    t_rm = ev_time(lambda i: w8.linear(xq, xsc, rm[i % 2][0], rm[i % 2][1], want_bf16=False,
                                       y_f32=lg, workspace=wsp))
    t_tl = ev_time(lambda i: w8.linear(xq, xsc, copies[i % 2][0], copies[i % 2][1],
                                       want_bf16=False, y_f32=lg, workspace=wsp))
    b = lm_head_bytes(M, V, K)
    res["lm_head_layouts_m5"] = {"tiled_us": round(t_tl * 1e6, 2),
                                 "tiled_GBs": round(b / t_tl / 1e9, 1),
                                 "row_major_us": round(t_rm * 1e6, 2),
                                 "row_major_GBs": round(b / t_rm / 1e9, 1)}
    # bf16 reference at the LM-head shape (two-times weight traffic), on the
    # tiled bf16 layout (each weight load one KiB, as for the int8 weights)
    # and, for context, on row-major bf16 weights
    t_bf_rm = ev_time(lambda i: w8.bf16_linear(x_dev[0], rm[i % 2][2], want_bf16=False, y_f32=lg))
    bt = [w8.tile_weight_bf16(rm[i][2]) for i in range(2)]
    t_bf = ev_time(lambda i: w8.bf16_linear(x_dev[0], bt[i % 2], N=V, want_bf16=False, y_f32=lg))
    bb = 2 * V * K + 2 * M * K + 4 * M * V
    res["bf16_reference_lm_head_m5"] = {"us": round(t_bf * 1e6, 2), "GBs": round(bb / t_bf / 1e9, 1),
                                        "layout": "tiled bf16",
                                        "row_major_us": round(t_bf_rm * 1e6, 2),
                                        "row_major_GBs": round(bb / t_bf_rm / 1e9, 1),
                                        "w8a8_tiled_us": round(t_tl * 1e6, 2),
                                        "w8a8_tiled_GBs": round(b / t_tl / 1e9, 1),
                                        "time_ratio_bf16_over_w8a8": round(t_bf / t_tl, 3),
                                        "byte_ratio_bf16_over_w8a8": round(bb / b, 3)}
    del rm, bt

    # stochastic verification at T = 1 on the same LM head: quantize_act ->
    # linear (fp32 logits) -> verify_sample, and verify_sample alone
    G, B = M - 1, 1
    r = synth.rng(synth.W_LM_HEAD, 40, 0)
    ua = torch.from_numpy(r.integers(0, 1 << 32, size=(B, G), dtype=np.uint64)
                          .astype(np.uint32).view(np.int32)).to(dev)
    us = torch.from_numpy(r.integers(0, 1 << 64, size=B, dtype=np.uint64).view(np.int64)).to(dev)
    draft = torch.from_numpy(synth.draft_ids(synth.W_LM_HEAD, B, G, V)).to(dev)
    al = torch.empty(B, dtype=torch.int32, device=dev)
    nt = torch.empty(B, dtype=torch.int32, device=dev)

    def stoch_step(i):
        w8.quantize_act(x_dev[i % len(x_dev)], xq=xq, x_scale=xsc)
        w8.linear(xq, xsc, copies[i % 2][0], copies[i % 2][1], want_bf16=False, y_f32=lg,
                  workspace=wsp)
        w8.verify_sample(lg, draft, 1.0, ua, us, accept_len=al, next_token=nt, workspace=wsp)

    t_st = graph_time([lambda: stoch_step(0), lambda: stoch_step(1)], replays=50) / 2
    t_vs = graph_time([lambda: w8.verify_sample(lg, draft, 1.0, ua, us, accept_len=al,
                                                next_token=nt, workspace=wsp)] * 8,
                      replays=50) / 8
    res["batched_verify_step_m288"] = batched_verify_measurement(dev, copies, wsp)
    res["w4a8_lm_head_m5"] = w4a8_measurement(dev, x_dev, xq, xsc, wsp)
    res["qwen3_8b_layer_step_m5"] = layer_step_measurement(dev, wsp)
    res["attention_scaling"] = attention_scaling(dev)

    # the online smoothing multiply fused into quantize_act, on the outlier
    # activations of the layer inputs: 16 launches per graph over 16 inputs
    sm = {}
    for Mq, Kq in ((5, 4096), (5, 12288), (8, 25600)):
        xs_l = [torch.from_numpy(synth.activations_bf16(synth.W_LAYER_M5, Mq, Kq, index=i,
                                                        outliers=True).view(np.int16).copy())
                .view(torch.bfloat16).to(dev) for i in range(16)]
        svec = torch.from_numpy(synth.smoothing_vector(synth.W_LAYER_M5, Kq)).to(dev)
        oq = torch.empty(Mq, Kq, dtype=torch.int8, device=dev)
        osc = torch.empty(Mq, dtype=torch.float32, device=dev)
        t_plain = graph_time([(lambda i=i: w8.quantize_act(xs_l[i], xq=oq, x_scale=osc))
                              for i in range(16)], replays=20) / 16
        t_smooth = graph_time([(lambda i=i: w8.quantize_act(xs_l[i], svec, xq=oq, x_scale=osc))
                               for i in range(16)], replays=20) / 16
        sm[f"M{Mq}_K{Kq}"] = {"plain_us": round(t_plain * 1e6, 2),
                              "smoothed_us": round(t_smooth * 1e6, 2)}
    res["quantize_act_smoothing_cost"] = sm
    res["stochastic_step_m5_t1"] = {
        "ms_per_step": round(t_st * 1e3, 5), "verified_tokens_per_s": round(M / t_st, 1),
        "verify_sample_us": round(t_vs * 1e6, 2),
        "verify_sample_logit_GBs": round(4 * M * V / t_vs / 1e9, 1),
        "step": "quantize_act + LM-head linear (fp32 logits) + verify_sample (T=1)",
        "timing": "HIP graph, 2 weight copies alternating; verify_sample alone: 8 launches"}
    return res


def stack32b_measurement(dev, wsp, replays=10):
    """The Qwen3-32B-shaped linear stack at M = 8 (7 drafts + 1): 64 layers
    of q/k/v/o/gate/up/down plus the LM head 5120 -> 151936, int8 weights
    (32 GB, tiled layout) drawn on the device, and the matching bf16 stack
    (64 GB) run through the in-build bf16 GEMM as the two-times-traffic
    reference.  q/k/v and gate/up are stored fused: each layer holds one
    [q;k;v] and one [gate;up] weight (their output channels stacked; per-
    channel quantization makes the codes and scales those of the separate
    matrices), so one launch covers each group.  One step: per layer,
    quantize_act of its four distinct inputs and its linears; then
    quantize_act, the LM head with the argmax folded in, and greedy
    acceptance (bf16: the LM head's fp32 logits, then verify_accept).  The
    stack never fits the 256 MB Infinity Cache, so no rotation is needed.
    Each step is one HIP graph replay; the layer inputs are seeded synthetic
    activations (no decoder-layer glue between the linears).  The same step
    is also timed with the seven linears launched separately (views into
    the fused weights)."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    M, G = 8, 7
    L = synth.QWEN3_32B_LAYERS
    lins = synth.QWEN3_32B_LAYER
    head = synth.QWEN3_32B_LM_HEAD
    groups = ((0, 1, 2), (3,), (4, 5), (6,))   # [q;k;v], o, [gate;up], down
    t0 = time.perf_counter()
    wts = []     # per layer, per group: (wq tiled, w_scale, w bf16)
    for layer in range(L):
        row = []
        for grp in groups:
            w = torch.cat([synth.weights_device(synth.W_STACK32B,
                                                synth.stack_tensor_index(layer, li),
                                                lins[li].N, lins[li].K, dev) for li in grp])
            wq, ws = w8.quantize_weight(w, tiled=True)
            row.append((wq, ws, w8.tile_weight_bf16(w.to(torch.bfloat16))))
            del w
        wts.append(row)
    lm = make_weight(head.N, head.K, synth.W_STACK32B, synth.stack_tensor_index(L, 0), dev,
                     tiled=True, with_bf16="tiled")
    torch.cuda.synchronize()
    print(f"[bench] 32B stack drawn and quantized on the device "
          f"({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)

    def act(K, index, layer):
        b = synth.activations_bf16(synth.W_STACK32B, M, K, index=index, outliers=True, layer=layer)
        return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(dev)

    in_k = tuple(lins[g[0]].K for g in groups)
    xs = [[act(k, 10_000 + 4 * layer + j, layer) for j, k in enumerate(in_k)] for layer in range(L)]
    x_lm = act(head.K, 20_000, L)
    xq = {k: torch.empty(M, k, dtype=torch.int8, device=dev) for k in set(in_k) | {head.K}}
    xsc = torch.empty(M, dtype=torch.float32, device=dev)
    ys = [torch.empty(M, sum(lins[li].N for li in g), dtype=torch.bfloat16, device=dev)
          for g in groups]
    draft = torch.from_numpy(synth.draft_ids(synth.W_STACK32B, 1, G, head.N)).to(dev)
    am = torch.empty(M, dtype=torch.int32, device=dev)
    al = torch.empty(1, dtype=torch.int32, device=dev)
    nt = torch.empty(1, dtype=torch.int32, device=dev)
    logits = torch.empty(M, head.N, dtype=torch.float32, device=dev)

    # the separate linears: row ranges of the fused weights (whole 16-row tiles)
    parts = []
    for layer in range(L):
        pl = []
        for j, grp in enumerate(groups):
            wq, ws, _ = wts[layer][j]
            n0 = 0
            for li in grp:
                n = lins[li].N
                pl.append((wq[n0 // 16:(n0 + n) // 16], ws[n0:n0 + n]))
                n0 += n
        parts.append(pl)
    ysep = [torch.empty(M, lin.N, dtype=torch.bfloat16, device=dev) for lin in lins]

    def head_step():
        w8.quantize_act(x_lm, xq=xq[head.K], x_scale=xsc)
        w8.lm_head_argmax(xq[head.K], xsc, lm[0], lm[1], workspace=wsp)
        w8.accept_from_keys(draft, argmax=am, accept_len=al, next_token=nt, workspace=wsp)

    def w8a8_step():
        for layer in range(L):
            for j, k in enumerate(in_k):
                w8.quantize_act(xs[layer][j], xq=xq[k], x_scale=xsc)
                wq, ws, _ = wts[layer][j]
                w8.linear(xq[k], xsc, wq, ws, y_bf16=ys[j], workspace=wsp)
        head_step()

    def w8a8_step_separate():
        for layer in range(L):
            pl = iter(parts[layer])
            for j, k in enumerate(in_k):
                w8.quantize_act(xs[layer][j], xq=xq[k], x_scale=xsc)
                for li in groups[j]:
                    wq, ws = next(pl)
                    w8.linear(xq[k], xsc, wq, ws, y_bf16=ysep[li], workspace=wsp)
        head_step()

    def bf16_step():
        for layer in range(L):
            for j in range(4):
                w8.bf16_linear(xs[layer][j], wts[layer][j][2], N=ys[j].shape[1], y_bf16=ys[j])
        w8.bf16_linear(x_lm, lm[2], N=head.N, want_bf16=False, y_f32=logits)
        w8.verify_accept(logits, draft, argmax=am, accept_len=al, next_token=nt, workspace=wsp)

    t_w8 = graph_time([w8a8_step], replays=replays)
    t_sep = graph_time([w8a8_step_separate], replays=replays)
    t_bf = graph_time([bf16_step], replays=replays)
    w8_bytes = L * sum(linear_bytes(M, lin.N, lin.K) for lin in lins) + \
        L * sum(M * k + 4 * M for k in in_k) + lm_head_bytes(M, head.N, head.K, logits=False)
    bf_bytes = L * sum(2 * lin.N * lin.K + 2 * M * lin.K + 2 * M * lin.N for lin in lins) + \
        2 * head.N * head.K + 2 * M * head.K + 4 * M * head.N
    weight_bytes = L * sum(lin.N * lin.K for lin in lins) + head.N * head.K
    res = {"M": M, "G": G, "layers": L, "int8_weight_bytes": weight_bytes,
           "w8a8_ms_per_step": round(t_w8 * 1e3, 4),
           "w8a8_verified_tokens_per_s": round(M / t_w8, 1),
           "w8a8_GBs": round(w8_bytes / t_w8 / 1e9, 1),
           "w8a8_frac_of_peak": round(w8_bytes / t_w8 / 1e9 / HBM_PEAK_GBS, 4),
           "w8a8_separate_linears_ms_per_step": round(t_sep * 1e3, 4),
           "bf16_ms_per_step": round(t_bf * 1e3, 4),
           "bf16_verified_tokens_per_s": round(M / t_bf, 1),
           "bf16_GBs": round(bf_bytes / t_bf / 1e9, 1),
           "time_ratio_bf16_over_w8a8": round(t_bf / t_w8, 3),
           "timing": f"HIP graph of one whole step, mean of {replays} replays",
           "launches_per_step": L * 8 + 3,
           "weights": "q/k/v and gate/up fused per layer (one launch each)"}
    del wts, lm, parts
    torch.cuda.empty_cache()
    return res


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return os.cpu_count() or 1


def _one_thread():
    """Context that holds every BLAS / OpenMP pool of this process to one
    thread (the oracle's elementwise numpy steps are single-threaded
    anyway)."""
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=1)


def oracle_timings():
    """The oracle's time for the other workloads' steps on this host (a
    reported baseline beside the GPU figures, never a target): per linear,
    quantize_act + the exact int product + dequant on random int8 codes of
    the workload's shapes (the codes do not change the oracle's work).  Each
    linear runs once untimed first (page faults, BLAS start-up), then is
    timed on all BLAS threads and again on one thread.  The 32B stack is
    timed as one layer plus the LM head and extrapolated to 64 layers."""
    import numpy as np

    import oracle
    import synth
    blas = _blas_threads()
    r = np.random.default_rng([9, 9, 9])

    def lin_times(M, N, K):
        xbits = synth.activations_bf16(99, M, K)
        wq = r.integers(-127, 128, size=(N, K), dtype=np.int8)
        ws = r.uniform(1e-4, 1e-3, N).astype(np.float32)

        def once():
            t0 = time.perf_counter()
            xq, xs = oracle.quantize_act(xbits)
            oracle.w8a8_linear(xq, xs, wq, ws)
            return time.perf_counter() - t0

        once()                                  # warm-up, untimed
        t_all = once()
        with _one_thread():
            t_one = once()
        return t_all, t_one

    out = {"kind": "oracle", "blas_threads": blas, "host_cores": len(os.sched_getaffinity(0)),
           "what": "all = every BLAS thread; one = BLAS held to one thread; warm-up call untimed"}
    for name, M in (("qwen3_8b_layer_linears_m5", 5), ("qwen3_8b_layer_linears_m288", 288)):
        per = {l.name: lin_times(M, l.N, l.K) for l in synth.QWEN3_8B_LAYER}
        out[name] = {"per_linear_ms": {k: round(v[0] * 1e3, 2) for k, v in per.items()},
                     "per_linear_ms_one_thread": {k: round(v[1] * 1e3, 2) for k, v in per.items()},
                     "sum_ms": round(sum(v[0] for v in per.values()) * 1e3, 2),
                     "sum_ms_one_thread": round(sum(v[1] for v in per.values()) * 1e3, 2)}
    layer = [lin_times(8, l.N, l.K) for l in synth.QWEN3_32B_LAYER]
    head = synth.QWEN3_32B_LM_HEAD
    head_t = lin_times(8, head.N, head.K)
    res = {}
    for k, tag in ((0, ""), (1, "_one_thread")):
        layer_s = sum(t[k] for t in layer)
        step_s = 64 * layer_s + head_t[k]
        res.update({f"one_layer_ms{tag}": round(layer_s * 1e3, 1),
                    f"lm_head_ms{tag}": round(head_t[k] * 1e3, 1),
                    f"step_ms_extrapolated_x64{tag}": round(step_s * 1e3, 1),
                    f"verified_tokens_per_s_extrapolated{tag}": round(8 / step_s, 3)})
    out["qwen3_32b_stack_m8"] = res
    return out


def library_int8_gemm(dev):
    """Context for the 288-row linears: the vendor int8 GEMM behind
    torch._int_mm (int8 x int8 -> int32, no scales, no epilogue) at the same
    shapes, weights rotated past the Infinity Cache as for ours.  Not part of
    the verification path."""
    import torch
    out = {}
    for name, M, N, K in (("q", 288, 4096, 4096), ("gate", 288, 12288, 4096),
                          ("down", 288, 4096, 12288), ("gate_up", 288, 24576, 4096)):
        g = torch.Generator(device=dev)
        g.manual_seed(11)
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
        ncp = max(2, int(600e6 // (N * K)) + 1)
        ws = [torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g)
              for _ in range(ncp)]
        try:
            t = graph_time([(lambda c=c: torch._int_mm(a, ws[c].t())) for c in range(ncp)],
                           replays=10) / ncp
            out[name] = {"us": round(t * 1e6, 2), "TOPS": round(2 * M * N * K / t / 1e12, 1)}
        except Exception as e:   # the op is missing or unsupported in the library
            out[name] = {"error": str(e)[:160]}
        del ws
        torch.cuda.empty_cache()
    out["what"] = "torch._int_mm (vendor int8 GEMM, int32 out, no dequant), HIP graph"
    # and the vendor bf16 GEMM on the M = 5 LM head (the 2x-traffic baseline
    # our own bf16 kernel also measures)
    g = torch.Generator(device=dev)
    g.manual_seed(12)
    x = torch.randn(5, 4096, device=dev, generator=g).to(torch.bfloat16)
    ws = [(torch.randn(151936, 4096, device=dev, generator=g) * 0.02).to(torch.bfloat16)
          for _ in range(2)]
    t = graph_time([(lambda c=c: torch.matmul(x, ws[c].t())) for c in range(2)], replays=10) / 2
    out["bf16_lm_head_m5"] = {"us": round(t * 1e6, 2),
                              "GBs": round(2 * 151936 * 4096 / t / 1e9, 1),
                              "what": "torch.matmul bf16, M=5, K=4096, N=151936"}
    del ws
    torch.cuda.empty_cache()
    return out


def attention_scaling(dev):
    """verify_attention alone over growing caches: Qwen3-8B heads (32 / 8)
    at T = 5 and Qwen3-32B heads (64 / 8) at T = 8, one sequence, and 32
    sequences of 4096 positions.  Two caches alternate inside a HIP graph;
    GB/s counts the K and V bytes the call must read."""
    import torch

    import w8a8_quantized_verification_amd as w8

    out = []
    # (adjacent workloads launch different grids: the trace summary splits on that)
    for (B, T, Hq, Hkv, ctx) in ATTENTION_WORKLOADS:
        g = torch.Generator(device=dev)
        g.manual_seed(77)
        caches = []
        for _ in range(2):
            kv = torch.randn(2, B, Hkv, ctx, 128, device=dev, generator=g).to(torch.bfloat16)
            caches.append((kv[0].contiguous(), kv[1].contiguous()))
            del kv
        q = torch.randn(B, T, Hq, 128, device=dev, generator=g).to(torch.bfloat16)
        lengths = torch.full((B,), ctx, dtype=torch.int32, device=dev)
        ws = w8.Workspace()
        o = torch.empty_like(q)
        t = graph_time([(lambda c=c: w8.verify_attention(q, *caches[c], lengths, out=o,
                                                         workspace=ws)) for c in range(2)],
                       replays=20) / 2
        kvb = 2 * B * Hkv * ctx * 128 * 2
        out.append({"B": B, "T": T, "Hq": Hq, "Hkv": Hkv, "positions": ctx,
                    "us": round(t * 1e6, 2), "kv_GBs": round(kvb / t / 1e9, 1),
                    "kv_frac_of_peak": round(kvb / t / 1e9 / HBM_PEAK_GBS, 4)})
        del caches
        torch.cuda.empty_cache()
    return out


def layer_step_measurement(dev, wsp, reps_copies=4, ctx=4096):
    """One Qwen3-8B decoder-layer step at M = 5 (one sequence, 4 drafts + 1)
    entirely through the library: residual + RMSNorm + quant -> [q;k;v]
    linear -> per-head q/k norms + RoPE + KV-cache append -> attention over
    4096 cached positions -> quant -> o linear -> residual + RMSNorm + quant
    -> [gate;up] linear -> SwiGLU + quant -> down linear (11 launches).  4
    distinct layers' weights and caches rotate (775 MB of weights, past the
    Infinity Cache).  Also attention alone."""
    import numpy as np
    import torch

    import synth
    import w8a8_quantized_verification_amd as w8

    M, D, F, Hq, Hkv, Dh = 5, 4096, 12288, 32, 8, 128
    lins = synth.QWEN3_8B_LAYER
    groups = ((0, 1, 2), (3,), (4, 5), (6,))
    layers, caches = [], []
    for c in range(reps_copies):
        row = []
        for j, grp in enumerate(groups):
            w = torch.cat([synth.weights_device(synth.W_LAYER_M5, 5000 + 10 * c + li,
                                                lins[li].N, lins[li].K, dev) for li in grp])
            row.append(w8.quantize_weight(w, tiled=True))
            del w
        layers.append(row)
        kv = torch.randn(2, 1, Hkv, ctx, Dh, device=dev, generator=torch.Generator(device=dev)
                         .manual_seed(900 + c)).to(torch.bfloat16)
        caches.append((kv[0].contiguous(), kv[1].contiguous()))

    def bf(x):
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(dev)

    h = bf(synth.activations_bf16(synth.W_LAYER_M5, M, D, index=50))
    gamma = bf(synth.to_bf16_bits(np.ones(D, dtype=np.float32)))
    head_gamma = bf(synth.to_bf16_bits(np.ones(Dh, dtype=np.float32)))
    lengths = torch.full((1,), ctx, dtype=torch.int32, device=dev)
    y_qkv = torch.zeros(M, (Hq + 2 * Hkv) * Dh, dtype=torch.bfloat16, device=dev)
    qbuf = torch.empty(1, M, Hq, Dh, dtype=torch.bfloat16, device=dev)
    attn = torch.empty(1, M, Hq, Dh, dtype=torch.bfloat16, device=dev)
    y_o = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    y_gu = torch.empty(M, 2 * F, dtype=torch.bfloat16, device=dev)
    y_down = torch.zeros(M, D, dtype=torch.bfloat16, device=dev)
    xq_d = torch.empty(M, D, dtype=torch.int8, device=dev)
    xq_f = torch.empty(M, F, dtype=torch.int8, device=dev)
    xs = torch.empty(M, dtype=torch.float32, device=dev)
    awsp = w8.Workspace()

    def layer(c):
        L = layers[c]
        kc, vc = caches[c]
        w8.residual_rmsnorm_quant(h, gamma, 1e-6, delta=y_down, h_out=h, xq=xq_d, x_scale=xs)
        w8.linear(xq_d, xs, *L[0], y_bf16=y_qkv, workspace=wsp)
        w8.qk_norm_rope_append(y_qkv, head_gamma, head_gamma, lengths, kc, vc, T=M, Hq=Hq,
                               Hkv=Hkv, q_out=qbuf)
        w8.verify_attention(qbuf, kc, vc, lengths, out=attn, workspace=awsp)
        w8.quantize_act(attn.view(M, D), xq=xq_d, x_scale=xs)
        w8.linear(xq_d, xs, *L[1], y_bf16=y_o, workspace=wsp)
        w8.residual_rmsnorm_quant(h, gamma, 1e-6, delta=y_o, h_out=h, xq=xq_d, x_scale=xs)
        w8.linear(xq_d, xs, *L[2], y_bf16=y_gu, workspace=wsp)
        w8.silu_mul_quant(y_gu[:, :F], y_gu[:, F:], xq=xq_f, x_scale=xs)
        w8.linear(xq_f, xs, *L[3], y_bf16=y_down, workspace=wsp)

    t = graph_time([(lambda c=c: layer(c)) for c in range(reps_copies)], replays=20) / reps_copies
    t_att = graph_time([(lambda c=c: w8.verify_attention(qbuf, *caches[c], lengths, out=attn,
                                                         workspace=awsp))
                        for c in range(reps_copies)], replays=20) / reps_copies
    wbytes = sum(l.N * l.K for l in lins)
    kvbytes = 2 * Hkv * ctx * Dh * 2
    res = {"M": M, "context": ctx, "us_per_layer": round(t * 1e6, 2),
           "weight_GBs": round(wbytes / t / 1e9, 1),
           "weight_plus_kv_GBs": round((wbytes + kvbytes) / t / 1e9, 1),
           "weight_plus_kv_frac_of_peak": round((wbytes + kvbytes) / t / 1e9 / HBM_PEAK_GBS, 4),
           "attention_us": round(t_att * 1e6, 2),
           "attention_kv_GBs": round(kvbytes / t_att / 1e9, 1),
           "launches": 12,
           "step": "rmsnorm+quant, qkv, q/k norm+rope+kv append, attention (2 kernels), quant, "
                   "o, rmsnorm+quant, gate_up, swiglu+quant, down"}
    del layers, caches
    return res


def cpu_baseline(w_host, xs_host, drafts, seconds, M):
    """The oracle's verify step on this host's cores, on a bounded sample of
    the 1000-trial LM-head workload (M=5, K=4096, V=151936): whole steps
    (quantize_act, the exact int8 product, dequant, argmax, acceptance) of
    trials 0, 1, 2, ... until ``seconds`` have passed (at least 2, at most
    100), first with every BLAS thread, then with BLAS held to one thread
    for about half as long.  The oracle quantizes the weights itself
    (untimed) from the same fp32 draw as the GPU copies, and one step runs
    untimed first."""
    import oracle
    wq, ws = oracle.quantize_weight(w_host)
    blas = _blas_threads()
    host_cores = len(os.sched_getaffinity(0))

    def one_step(t):
        xq, xs = oracle.quantize_act(xs_host[t % len(xs_host)])
        _, y32, _ = oracle.w8a8_linear(xq, xs, wq, ws)
        oracle.verify_accept(y32, drafts[t % len(drafts)][None, :])

    def run(limit_s):
        t0 = time.perf_counter()
        steps = 0
        while steps < 100 and (steps < 2 or time.perf_counter() - t0 < limit_s):
            one_step(steps)
            steps += 1
        return steps, time.perf_counter() - t0

    one_step(0)                                   # warm-up, untimed
    steps, dt = run(seconds)
    with _one_thread():
        steps1, dt1 = run(seconds / 2)
    return {"value": round(M * steps / dt, 3), "unit": "verified tokens/s", "cores": blas,
            "kind": "oracle",
            "sample": f"{steps} LM-head verify steps (M=5, K=4096, V=151936; trials 0..{steps - 1} "
                      f"of the 1000-trial workload), numpy oracle, {dt:.1f} s after one untimed "
                      f"step; {blas} BLAS threads (elementwise steps single-threaded) on "
                      f"{host_cores} host cores",
            "host_cores": host_cores, "blas_threads": blas,
            "one_thread": {"value": round(M * steps1 / dt1, 3), "unit": "verified tokens/s",
                           "cores": 1, "steps": steps1, "seconds": round(dt1, 2)}}


if __name__ == "__main__":
    main()
