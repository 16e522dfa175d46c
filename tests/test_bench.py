"""Host-side pieces of bench.py (no GPU): the one-GPU guard, the counter
summary reader and the CPU-oracle baseline on a small workload."""

import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_kernel_sources_exist():
    for names in bench.KERNEL_SOURCES.values():
        for n in names:
            assert os.path.exists(os.path.join(ROOT, "branch_attention_speculative_amd", "csrc", n))


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCES))
def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(kernel, monkeypatch):
    path = os.path.join(ROOT, "profiles", f"{kernel}_long256k_traffic.md")
    txt = open(path).read()
    recorded = float(re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt).group(1))
    recorded_hash = re.search(r"source_hash:\s*([0-9a-f]+)", txt).group(1)
    # with the recorded hash the figure is used as is
    monkeypatch.setattr(bench, "source_hash", lambda names: recorded_hash)
    assert bench.read_traffic(kernel, "long256k") == recorded
    # any other source state gives no figure
    monkeypatch.setattr(bench, "source_hash", lambda names: "0" * 16)
    assert bench.read_traffic(kernel, "long256k") is None
    # and a workload without a summary gives none either
    assert bench.read_traffic(kernel, "no_such_workload") is None


def test_source_hash_tracks_file_contents():
    names = bench.KERNEL_SOURCES["bwd_dkdv"]
    h = bench.source_hash(names)
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    assert h == bench.source_hash(names)
    assert h != bench.source_hash(bench.KERNEL_SOURCES["fwd_ring"])


def test_cpu_baseline_on_the_tiny_workload():
    from oracle import pack
    w = workloads.make("tiny")
    lay = pack.zigzag_layout(w.seqlens, w.C, w.r)
    br = pack.branch_index(lay, w.kind, w.depth_or_block)
    counts = pack.pair_counts(lay, br)
    raw = workloads.draw(w, lay["n_local"], br["n_branch"])
    out = bench.cpu_baseline(w, {"pairs_total": counts["total"]}, raw, n_anchor_sample=5)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1
    # the sampled pairs are a part of the whole: 5 anchors' main rows and their
    # branch rows, each row's pairs counted from the visibility rules
    m = re.search(r"\((\d+) of (\d+) pairs per head", out["sample"])
    sampled, total = int(m.group(1)), int(m.group(2))
    assert total == counts["total"] and 0 < sampled < total
    assert out["extrapolated_step_s"] == pytest.approx(out["seconds"] * total / sampled)


def test_blended_peaks():
    """The fp8 forward's peak weighs Q K^T (fp8) and P V (bf16) equally; the
    fp8 step's counts 4 of its 14 D per pair at the fp8 rate: the time of a
    FLOP-weighted mix at each unit's own peak."""
    fp8, bf16 = bench.PEAK_FP8_TFLOPS, bench.PEAK_BF16_TFLOPS
    assert fp8 == pytest.approx(2 * bf16)
    assert bench.PEAK_FP8_QK_BF16_PV_TFLOPS == pytest.approx(4 * bf16 / 3)
    # 4 units at twice the rate and 10 at the base rate take 12 base-rate units
    assert bench.PEAK_FP8_STEP_TFLOPS == pytest.approx(14 * bf16 / 12)
    assert bench.PEAK_BF16_TFLOPS < bench.PEAK_FP8_STEP_TFLOPS < bench.PEAK_FP8_QK_BF16_PV_TFLOPS
