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


def test_cpu_baseline_compares_the_gpu_rows():
    """cpu_baseline's error fields: the oracle's own output (rounded to bf16)
    is within half a bf16 ulp, and a changed row shows up in the maxima."""
    import numpy as np
    import torch
    from dataclasses import replace
    from oracle import attention
    from workloads import make_inputs
    w = replace(WORKLOADS["bert_large"], B=1, H=2, N=300)
    q, k, v = make_inputs(w)
    o, lse = attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), w.scale)
    og, lg = torch.from_numpy(o).to(torch.bfloat16), torch.from_numpy(lse).float()
    r = bench.cpu_baseline(w, q, k, v, 30.0, og, lg)
    e = r["error_vs_oracle"]
    assert r["cores"] == len(os.sched_getaffinity(0)) and e["rows"] == 600
    assert e["o_max_abs"] <= 2.0 ** -8 * np.abs(o).max() and e["lse_max_abs"] < 1e-6
    og[0, 1, 17] += 0.5
    lg[0, 0, 5] += 0.01
    e = bench.cpu_baseline(w, q, k, v, 30.0, og, lg)["error_vs_oracle"]
    assert e["o_max_abs"] >= 0.49 and abs(e["lse_max_abs"] - 0.01) < 1e-4


def test_kernel_hash_ignores_comments_only():
    """The traffic counters stay tied to the kernel's code: editing a comment
    or blank lines keeps the hash, changing a token does not."""
    src = "int a = 1; // one\n/* block\n comment */\n\nint b = a + 2;\n"
    same = "int a = 1;   // another comment\n\n  int b = a + 2;  /* trailing */\n"
    other = "int a = 1;\nint b = a + 3;\n"
    assert bench._code_only(src) == bench._code_only(same)
    assert bench._code_only(src) != bench._code_only(other)


def test_warm_up_lasts_the_minimum_time(monkeypatch):
    """The warm-up runs the requested steps and then untimed launches until
    MIN_WARMUP_SECONDS have passed; the count is reported."""
    import time
    calls = []
    monkeypatch.setattr(bench, "MIN_WARMUP_SECONDS", 0.05)

    class FakeCuda:
        @staticmethod
        def synchronize():
            pass

    import torch
    monkeypatch.setattr(torch, "cuda", FakeCuda)
    t0 = time.perf_counter()
    bench.warm_up(lambda: calls.append(time.sleep(0.001)), 3)
    assert time.perf_counter() - t0 >= 0.05
    assert bench.WARMUP_RUN["launches"] == len(calls) > 3


def test_block_sparse_flop_count():
    """FLOPs of a block-sparse call: an all-ones mask counts the dense pairs
    (halved plus the diagonal when causal), an all-zeros mask none, and one
    set block its own clipped pairs (key <= query when causal)."""
    import dataclasses
    import numpy as np
    w = dataclasses.replace(WORKLOADS["patch_3mp"], B=1, H=1, N=300)
    wc = dataclasses.replace(w, causal=True)
    ones = np.ones((3, 5), dtype=bool)
    assert bench.sparse_flops(w, ones) == 4.0 * 300 * 300 * 64
    assert bench.sparse_flops(wc, ones) == 4.0 * (300 * 301 // 2) * 64
    assert bench.sparse_flops(w, np.zeros_like(ones)) == 0.0
    one = np.zeros_like(ones)
    one[2, 4] = True  # queries 256..299, keys 256..299
    assert bench.sparse_flops(w, one) == 4.0 * 44 * 44 * 64
    assert bench.sparse_flops(wc, one) == 4.0 * (44 * 45 // 2) * 64
    one = np.zeros_like(ones)
    one[0, 3] = True  # queries 0..127, keys 192..255: all above the diagonal
    assert bench.sparse_flops(wc, one) == 0.0
