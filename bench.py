#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

One step = one attn_fwd launch over the whole workload (all heads, all query
rows, all keys), inputs resident in device memory.  The default workload is
the 3 MP vision-decoder patch self-attention: B=1, H=16, N=11,616, d=64,
bf16, non-causal, scale 1/8.  Prints ONE JSON line on stdout; progress goes
to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--n N]
  python bench.py --sweep FILE   # one JSON line per workload into FILE

FLOPs per step are the algorithmic 4*B*H*N^2*d (QK^T plus PV), halved when
causal; exponentials are not counted.  The roofline peak is MI355X's
published dense bf16 MFMA rate (256 CUs x 4 SIMDs x 1024 flop/clk x 2.4 GHz).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "exact_attention_29_amd", "csrc", "attn_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak at H=16,d=64,P=11616"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(workload_name):
    """Measured HBM bytes per launch from committed rocprofv3 counter runs, or
    None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha():
        return None
    entry = t.get("workloads", {}).get(workload_name)
    if not entry:
        return None
    return entry["hbm_bytes_per_launch"]


def time_gpu(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall / steps, start.elapsed_time(end) * 1e-3 / steps


def cpu_baseline(w, q, k, v, seconds):
    """The fp64 oracle, as it stands, on a time-boxed sample of the same
    workload: the first query rows of head 0, 1, ... against all N keys."""
    import numpy as np
    from oracle import attention
    from workloads import to_f64
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        blas = 1
    chunk = 256
    rows_done, t0 = 0, time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            qf, kf, vf = (to_f64(t[b:b + 1, h:h + 1]) for t in (q, k, v))
            for r0 in range(0, w.N, chunk):
                rows = np.arange(r0, min(r0 + chunk, w.N))
                attention(qf, kf, vf, w.scale, causal=w.causal, rows=rows)
                rows_done += len(rows)
                if time.perf_counter() - t0 >= seconds:
                    break
            if time.perf_counter() - t0 >= seconds:
                break
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    if w.causal:
        flops = 0.0  # not used for the default workload
    else:
        flops = rows_done * w.N * w.d * 4.0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle on {rows_done} query rows x {w.N} keys of {w.name} "
                   f"({rows_done / (w.B * w.H * w.N):.2%} of the workload), {dt:.1f} s wall; "
                   f"matmuls on {blas} BLAS threads, exp single-threaded; "
                   f"host has {len(os.sched_getaffinity(0))} usable cores"),
    }


def bench_one(w, steps, warmup, with_cpu, cpu_seconds):
    import torch
    import exact_attention_29_amd as ea
    from workloads import make_inputs

    dev = "cuda:0"
    q, k, v = make_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    B, H, N, d = w.shape
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # workspace: extra device memory a call needs beyond its outputs
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    free0 = torch.cuda.mem_get_info(dev)[0]
    o_tmp, lse_tmp = ea.forward(qd, kd, vd, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    out_bytes = o_tmp.numel() * o_tmp.element_size() + lse_tmp.numel() * 4
    extra = torch.cuda.max_memory_allocated(dev) - base - out_bytes
    free_delta = free0 - torch.cuda.mem_get_info(dev)[0]
    del o_tmp, lse_tmp

    def step():
        ea.forward(qd, kd, vd, scale=w.scale, causal=w.causal, out=o, lse=lse)

    wall, kern = time_gpu(step, steps, warmup, stream)
    flops = w.flops
    value = flops / wall / 1e12
    achieved = flops / kern / 1e12
    traffic = traffic_for(w.name)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.what}",
            "B": B, "H": H, "N": N, "d": d, "causal": w.causal, "scale": w.scale,
            "inputs": f"i.i.d. N(0,{w.sigma}^2), seed {w.seed}",
            "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)",
        },
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "attn_fwd_bf16_kernel<%s>" % ("true, 4" if w.causal else "false, 8"),
            "kernel_ms": round(kern * 1e3, 4),
            "algorithmic_bytes": 4 * B * H * N * d * 2 + 4 * B * H * N,
        },
        "workspace": {"extra_bytes": int(extra), "mem_get_info_delta": int(free_delta),
                      "output_bytes": int(out_bytes)},
    }
    if with_cpu:
        log("[bench] timing the fp64 oracle on a sample ...")
        line["cpu_baseline"] = cpu_baseline(w, q, k, v, cpu_seconds)
    return line


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU clock ramps for ~60 launches (~35 ms) from idle; 100 untimed
    # warmup steps put the timed steps in steady state.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="patch_3mp")
    ap.add_argument("--n", type=int, default=None, help="override the sequence length")
    ap.add_argument("--causal", choices=["yes", "no"], default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--sweep", default=None, help="write one JSON line per workload to this file")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain elementwise copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the forward kernel has no multi-GPU path to measure.", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import PATCH_SWEEP, WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_mib:
        # A plain copy kernel of known size: reads and writes copy_mib MiB once.
        # rocprofv3's FETCH_SIZE / WRITE_SIZE for it give the counters' scale.
        n = args.copy_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "dispatches": 3}))
        return

    if args.sweep:
        cases = [WORKLOADS[n] for n in ("bert_large", "gpt2_small_causal")]
        cases += [WORKLOADS["patch_3mp"].with_n(n) for n in PATCH_SWEEP]
        cases += [WORKLOADS["patch_3mp"], WORKLOADS["patch_8mp"]]
        from dataclasses import replace
        cases.append(replace(WORKLOADS["patch_3mp"], causal=True, name="patch_3mp_causal"))
        with open(args.sweep, "w") as f:
            for w in cases:
                steps = max(args.steps, 200) if w.flops < 2e10 else args.steps
                warm = max(args.warmup, 1000) if w.flops < 2e10 else args.warmup
                log(f"[bench] {w.name} {w.shape} causal={w.causal}")
                line = bench_one(w, steps, warm, False, 0)
                f.write(json.dumps(line) + "\n")
                f.flush()
                log(f"[bench] {w.name}: {line['value']} TFLOP/s, kernel {line['roofline']['kernel_ms']} ms")
        return

    w = WORKLOADS[args.workload]
    if args.n:
        w = w.with_n(args.n)
    if args.causal:
        from dataclasses import replace
        w = replace(w, causal=args.causal == "yes")
    log(f"[bench] {w.name} {w.shape} {w.dtype} causal={w.causal} steps={args.steps} warmup={args.warmup}")
    line = bench_one(w, args.steps, args.warmup, not args.no_cpu_baseline, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
