"""bench.py's host logic without a GPU: the one-GPU refusal, the algorithmic
byte counts behind the roofline, the committed counter summary it reads (and
drops once the kernel source changes), and the kernel-trace ingest that
writes the profile summaries."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    env = dict(os.environ, WORLD_SIZE="1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_lm_head_bytes_are_the_operands_read_once():
    M, N, K = 5, 151936, 4096
    weights, w_scales, codes, x_scales = N * K, 4 * N, M * K, 4 * M
    assert bench.lm_head_bytes(M, N, K, logits=False) == weights + w_scales + codes + x_scales
    assert bench.lm_head_bytes(M, N, K) == weights + w_scales + codes + x_scales + 4 * M * N
    assert bench.linear_bytes(M, N, K) == weights + w_scales + codes + x_scales + 2 * M * N
    # the headline figure: 622.3 MB per launch, weights dominate
    assert 622_000_000 < bench.lm_head_bytes(M, N, K, logits=False) < 623_000_000


def test_committed_traffic_matches_the_kernel_source():
    """The counter summary under profiles/ was taken on the GEMM source in
    the tree (otherwise the bench line reports traffic as null), and its
    figure is close to the algorithmic bytes."""
    t = bench.read_traffic()
    assert t is not None, "profiles/gemm_w8a8_lm_head_m5_traffic.txt is stale: retake FETCH/WRITE_SIZE"
    alg = bench.lm_head_bytes(5, 151936, 4096, logits=False)
    assert 0.95 < t / alg < 1.10


def test_committed_batched_counters_match_the_kernel_source():
    """The 288-row counter summary (MfmaUtil, HBM traffic per shape) was
    taken on the batched kernels' source in the tree, and each shape's
    traffic is at least the algorithmic bytes."""
    c = bench.read_batched_counters()
    assert c is not None and not c["stale"], \
        "profiles/gemm_w8a8_batched_m288_counters.txt is stale: retake with --pmc-probe-batched"
    assert c["per_shape"]
    for shape, v in c["per_shape"].items():
        assert 0.0 < v["MfmaUtil"] < 100.0, shape
        assert v["hbm_over_algorithmic"] >= 0.99, shape


def test_traffic_is_dropped_for_another_kernel_source(tmp_path, monkeypatch):
    other = tmp_path / "gemm_w8a8.hip"
    other.write_text("// a different kernel source\n")
    monkeypatch.setattr(bench, "GEMM_SRC", str(other))
    assert bench.read_traffic() is None
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "absent.txt"))
    assert bench.read_traffic() is None


def test_ingest_trace_summarises_per_kernel(tmp_path):
    run = tmp_path / "trace" / "host"
    run.mkdir(parents=True)
    (run / "run_kernel_stats.csv").write_text(
        "Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs\n"
        "gemm_w8a8_skinny,3,300000,100000,90,90000,120000\n"
        "accept_keys_kernel,3,15000,5000,5,4000,6000\n")
    starts = [1_000_000, 2_000_000, 3_000_000]
    gemm = [90_000, 120_000, 90_000]     # median 90 us, mean 100
    acc = [4_000, 5_000, 6_000]
    lines = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    for s, g, a in zip(starts, gemm, acc):
        lines.append(f"gemm_w8a8_skinny,{s},{s + g}")
        lines.append(f"accept_keys_kernel,{s + 200_000},{s + 200_000 + a}")
    (run / "run_kernel_trace.csv").write_text("\n".join(lines) + "\n")
    out = tmp_path / "summary.txt"
    bench.ingest_trace(str(tmp_path / "trace"), "the command", str(out))
    text = out.read_text().splitlines()
    assert text[1] == "# command: the command"
    rows = {l.split()[-1]: [float(x) for x in l.split()[:4]] + [int(l.split()[4])] for l in text[3:]}
    assert rows["gemm_w8a8_skinny"] == [100.0, 90.0, 90.0, 120.0, 3]
    assert rows["accept_keys_kernel"] == [5.0, 5.0, 4.0, 6.0, 3]
