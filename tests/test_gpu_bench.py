"""bench.py end to end on the GPU, on the tiny workload: one JSON line with
the keys the measurement contract asks for."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_complete_json_line():
    torch = pytest.importorskip("torch")
    # device_count() does not initialise the GPU in this process; the bench
    # runs as a child process of its own
    if torch.cuda.device_count() < 1:
        pytest.skip("no GPU visible")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                          "--steps", "2", "--warmup", "1", "--cpu-anchors", "2",
                          "--mfma-probe-iters", "200"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2516.6
    assert r["achieved"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    p = d["mfma_probe"]
    assert p["zero_operands_tflops"] > 0 and p["random_operands_tflops"] > 0


def test_bench_fp8_step_with_the_backward():
    """--dtype fp8 --fp8-step fwd+bwd on the ttt32k workload: the
    backward runs (its kernels in the per-kernel table), the metric and peak
    are the fp8 step's, and the dominant kernel is priced at its own peak."""
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() < 1:
        pytest.skip("no GPU visible")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "ttt32k",
                          "--dtype", "fp8", "--fp8-step", "fwd+bwd", "--steps", "2", "--warmup", "1",
                          "--cpu-anchors", "0", "--mfma-probe-iters", "0"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    d = json.loads([l for l in res.stdout.splitlines() if l.strip()][-1])
    assert d["dtype"] == "fp8" and "fwd+bwd" in d["metric"]
    assert {"fwd_ring", "bwd_dq", "bwd_dkdv"} <= set(d["kernels"])
    assert d["split"]["bwd_ms"] > 0
    assert 2516.6 < 100.0 * d["value"] / d["pct_of_peak"] < 5033.2
    r = d["roofline"]
    assert r["kernel"] == "bwd_dkdv" and r["peak"] == 2516.6 and r["traffic"] is None
