"""The benchmark's host-side contract (no GPU): the one-GPU rule, the committed counter
summary it reads, and the oracle's CPU baseline leg."""
import json
import os
import subprocess
import sys

import bench
from workload import WORKLOADS, make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_summary_matches_its_workload():
    with open(os.path.join(ROOT, "profiles", "traffic_tile_kernel_fused_gpt2_mlp.json")) as f:
        d = json.load(f)
    w = WORKLOADS["gpt2_mlp"]
    assert d["algorithmic_bytes_per_launch"] == 2 * w.M * w.K + 2 * w.K * w.N + 6 * w.M * w.N + 2 * w.N
    assert d["traffic_bytes_per_launch"] == d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"]
    cal = d["calibration"]
    kib = cal["copy_bytes"] / 1024
    assert abs(cal["fetch_factor"] - kib / cal["fetch_size_kib"]) < 1e-3
    assert abs(cal["write_factor"] - kib / cal["write_size_kib"]) < 1e-3
    # the request-counter derivation: bytes are requests times their sizes, the copy of
    # 1 GiB reads and writes 1 GiB, and the fused kernel's figure agrees with the calibrated
    # one within the machine-to-machine spread
    rq = d["request_counters"]
    f = rq["fused"]
    assert f["read_bytes_per_launch"] == (128 * f["TCC_EA0_RDREQ_128B"] + 64 * f["TCC_EA0_RDREQ_64B"]
                                          + 32 * f["TCC_EA0_RDREQ_32B"])
    assert f["write_bytes_per_launch"] == (64 * f["TCC_EA0_WRREQ_64B"]
                                           + 32 * (f["TCC_EA0_WRREQ"] - f["TCC_EA0_WRREQ_64B"]))
    assert f["traffic_bytes_per_launch"] == f["read_bytes_per_launch"] + f["write_bytes_per_launch"]
    cp = rq["copy_1GiB"]
    assert abs(cp["read_bytes"] / cal["copy_bytes"] - 1) < 1e-3
    assert abs(cp["write_bytes"] / cal["copy_bytes"] - 1) < 1e-3
    assert abs(f["traffic_bytes_per_launch"] / d["traffic_bytes_per_launch"] - 1) < 0.03
    # the bench reports the counters only while they describe the current kernel sources
    t = bench._traffic(bench.tile_kernel_sha())
    assert t is None or t == d["traffic_bytes_per_launch"]
    assert bench._traffic("0" * 64) is None


def test_cpu_baseline_fields():
    w = WORKLOADS["tiny"]
    cb = bench._cpu_baseline(make_inputs("tiny"), w, budget_s=5.0)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert f"M={w.M}" in cb["sample"]
