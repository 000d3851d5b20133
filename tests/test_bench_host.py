"""Host-side contract of bench.py, on the CPU: the one-GPU refusal, the
measured-traffic lookup (reported only for the kernel source it was taken
on) and the FLOP count the throughput is quoted on."""

import json
import os
import subprocess
import sys

import bench
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr


def test_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    entry = {"hbm_bytes_per_launch": 123456789}
    f.write_text(json.dumps({"kernel_sha": bench.kernel_sha(), "workloads": {"patch_3mp": entry}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("patch_3mp") == 123456789
    assert bench.traffic_for("bert_large") is None
    f.write_text(json.dumps({"kernel_sha": "0" * 16, "workloads": {"patch_3mp": entry}}))
    assert bench.traffic_for("patch_3mp") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("patch_3mp") is None


def test_committed_traffic_figures_are_whole_launches():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    for name, e in t["workloads"].items():
        assert name in WORKLOADS
        # bytes read = 2 x FETCH_SIZE, written = WRITE_SIZE (KiB), as calibrated;
        # the KiB figures are stored rounded to 0.1 KiB
        total = (e["fetch_kib"] * t["fetch_scale"] + e["write_kib"] * t["write_scale"]) * 1024
        assert abs(e["hbm_bytes_per_launch"] - total) <= 0.05 * 1024 * (t["fetch_scale"] + t["write_scale"])


def test_flop_count():
    # 4 B H N^2 d: QK^T and PV, two flops per multiply-add; halved when causal
    w = WORKLOADS["patch_3mp"]
    assert w.flops == 4 * 1 * 16 * 11616 ** 2 * 64 == 552_679_243_776
    g = WORKLOADS["gpt2_small_causal"]
    assert g.flops == 2 * 8 * 12 * 1024 ** 2 * 64
