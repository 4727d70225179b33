"""bench.py's output contract: one JSON line with the step's throughput, the
dominant kernel against its roofline, and the CPU baseline; one GPU only.

The CPU tests check the argument handling and the committed counter summary
that `roofline.traffic` comes from; the GPU test runs a short benchmark and
checks every field of its line.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_committed_traffic_summary_is_consistent():
    sys.path.insert(0, ROOT)
    import bench
    t = json.load(open(bench.TRAFFIC_FILE))
    assert t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"] == pytest.approx(t["hbm_bytes_per_launch"], abs=2)
    # the fused kernel reads q8, k8, V and the scales and writes O: HBM traffic cannot be below that
    assert t["hbm_bytes_per_launch"] >= 0.99 * t["algorithmic_bytes_per_launch"]
    assert len(t["kernel_source_digest"]) == 16
    # bench.py reports the traffic only while the kernel source is the one the counters were taken on
    got = bench.traffic_or_null()
    assert got is None or got == t["hbm_bytes_per_launch"]


@pytest.mark.gpu
def test_bench_line_fields():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[bench] --steps 3 --warmup 1 --no-extra --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, "-u", BENCH, "--steps", "3", "--warmup", "1", "--no-extra",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "TOPS" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 5000.0
    assert rf["achieved"] > 0 and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    assert rf["traffic"] is None or rf["traffic"] > 0
    # value counts both passes of the step; a step holds at least the two kernel launches it times
    assert d["ms_per_step"] >= rf["kernel_ms"] + rf["causal_kernel_ms"]
