"""bench.py's host side, on the CPU: the one-GPU contract and the rule that
profiled figures (counters, HBM traffic) are reported only for the kernel
source they were taken on.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

WORKLOADS = ["wide_m5_k4", "wide_m8_k3", "wide_m15_k2", "down_m15_k4", "matvec_m1_k4", "gateup_m5_k4",
             "packed_3x5_k4"]


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for an unmeasured configuration


@pytest.mark.parametrize("w", WORKLOADS)
def test_figures_are_reported_only_for_their_source(w):
    # With the summaries' own source hash the figures come back; with any
    # other (the kernel changed since they were taken) they are withheld.
    with open(os.path.join(ROOT, "profiles", f"counters_prefill_{w}.json")) as f:
        sha = json.load(f)["kernel_sha"]
    fig = bench.profile_figures(w, sha)
    assert fig is not None and 0.0 < fig["valu_busy_profiled"] <= 1.0 and fig["valu_ops_per_weight_profiled"] > 0
    with open(os.path.join(ROOT, "profiles", f"traffic_prefill_{w}.json")) as f:
        tsha = json.load(f)["kernel_sha"]
    assert bench.traffic_from_profiles(w, tsha) > 0
    assert bench.profile_figures(w, "0" * 16) is None
    assert bench.traffic_from_profiles(w, "0" * 16) is None
