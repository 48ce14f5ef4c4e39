"""The benchmark's output contract on the GPU, in this process: one short
run of bench.main (20 timed steps, no extras, a 2 s CPU sample) prints one
JSON line with the keys its readers use, every timed verdict equal to the
oracle's, a roofline whose achieved figure follows from its own byte count
and launch time, and the oracle's CPU baseline."""
import json
import sys

import pytest

from tests.gpu_util import announce, gpu_available

pytestmark = pytest.mark.gpu

KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
        "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
        "roofline", "cpu_baseline")


def test_bench_json_line(capsys, monkeypatch):
    if not gpu_available():
        pytest.skip("no ROCm GPU")
    import bench
    announce("bench.main --steps 20 --warmup 5 --no-extra --cpu-seconds 2")
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "20", "--warmup", "5", "--no-extra",
                                      "--cpu-seconds", "2"])
    capsys.readouterr()
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for k in KEYS:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5
    assert d["higher_is_better"] is True and d["dtype"] == "int8"
    assert d["config"]["workload"] == "lm_head_verify_m5"
    M = d["config"]["M"]
    assert abs(d["value"] - M / (d["ms_per_step"] * 1e-3)) <= 0.01 * d["value"]
    assert d["verdicts_match_oracle"] == "20/20"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    derived = roof["algorithmic_bytes_per_launch"] / (roof["avg_launch_us"] * 1e-6) / 1e9
    assert abs(roof["achieved"] - derived) <= 0.01 * roof["achieved"]
    assert 0.3 < roof["frac"] < 1.0
    assert roof["traffic"] is not None and roof["achievable"] > roof["achieved"] * 0.8
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
