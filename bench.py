#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

One step = one attn_fwd launch over the whole workload (all heads, all query
rows, all keys), inputs resident in device memory.  The default workload is
the 3 MP vision-decoder patch self-attention: B=1, H=16, N=11,616, d=64,
bf16, non-causal, scale 1/8.  Prints ONE JSON line on stdout; progress goes
to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--n N]
  python bench.py --sweep FILE   # one JSON line per workload into FILE
  python bench.py --workspace-sweep   # device memory beyond O and LSE vs P, with fits
  python bench.py --backward [--key-len L | --key-density D | --block-density D] [--layout packed]   # dQ, dK, dV instead

Besides the contract fields, the line carries per-launch kernel time (mean,
median, min) from HIP events on the launch stream, a cold-cache variant
(caches flushed by rewriting a 512 MiB buffer before each launch), the shader
clock sampled with amd-smi and the roofline fraction at that clock, the
workspace a call needs, and the fp64 oracle timed on a sample on the host.

FLOPs per step are the algorithmic 4*B*H*N^2*d (QK^T plus PV), halved when
causal; exponentials are not counted.  The roofline peak is MI355X's
published dense bf16 MFMA rate (256 CUs x 4 SIMDs x 1024 flop/clk x 2.4 GHz).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
KERNEL_SRCS = [os.path.join(ROOT, "exact_attention_29_amd", "csrc", f) for f in ("attn_fwd.hip", "attn_common.h", "attn_split.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak at H=16,d=64,P=11616"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text):
    """C++ source without comments and blank lines, each line stripped: the
    part of the source that decides the compiled kernel."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.strip() for line in text.splitlines() if line.strip())


def kernel_sha():
    """Hash of the forward kernel's sources, comments and whitespace left out
    (the traffic counters are only reported for the code they were taken
    on; a comment edit does not change the kernel)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def library_splits(B, H, N, cus):
    """Whether attn_fwd_split splits the last round of a non-causal call
    (the library's rule, restated: 256-row tiles dealt to 8 XCDs of C = cus/8
    CUs; split when the tiles left past the whole rounds fill at most half a
    round, there is a whole round before them or the rows have at least 160
    key tiles, no XCD's leftover is a whole round, the rows are at least
    64*C keys long, and C*C*ceil(N/64) < 2^31)."""
    c = cus // 8 if cus >= 16 else 1
    tiles = B * H * -(-N // 256)
    n_kt = -(-N // 64)
    per, r8 = divmod(tiles, 8)
    rounds = per // c
    rem_max = per + (1 if r8 else 0) - rounds * c
    left = tiles - 8 * rounds * c
    return (0 < rem_max < c and n_kt >= c and 2 * left <= 8 * c and (rounds >= 1 or n_kt >= 160)
            and c * c * n_kt < 2 ** 31 and c <= 64)


def kernel_name(w, B, H, N, sparse, bit_mask, split=True):
    """The forward kernel instantiation a call runs (the library's choice:
    block-sparse and causal calls 4 waves; non-causal through
    attn_fwd_split the split 8-wave kernel when library_splits, else 8
    waves when B*H*ceil(N/256) reaches the CU count, else 4)."""
    import torch
    mask = "true" if bit_mask else "false"
    if sparse:
        return "attn_fwd_bf16_kernel<%s, 4, false, true, false>" % ("true" if w.causal else "false")
    if w.causal:
        return "attn_fwd_bf16_kernel<true, 4, %s, false, false>" % mask
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if split and library_splits(B, H, N, cus):
        return "attn_fwd_bf16_kernel<false, 8, %s, false, true>" % mask
    waves = 8 if B * H * ((N + 255) // 256) >= cus else 4
    return "attn_fwd_bf16_kernel<false, %d, %s, false, false>" % (waves, mask)


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


# From idle the shader clock takes ~60 launches of the 3 MP kernel (~35 ms)
# to ramp up; after the requested warm-up steps, untimed launches (graph
# replays, for the graph timer) continue until the warm-up has kept the GPU
# busy this long, so the timed steps see the steady state however few
# warm-up steps were asked for.
MIN_WARMUP_SECONDS = 0.5
WARMUP_RUN = {"launches": 0}


def warm_up(fn, warmup):
    """The requested warm-up steps, then more untimed launches until
    MIN_WARMUP_SECONDS have passed; the count run is kept in WARMUP_RUN."""
    import torch
    t0 = time.perf_counter()
    n = 0
    for _ in range(warmup):
        fn()
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < MIN_WARMUP_SECONDS:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    WARMUP_RUN["launches"] = n


def time_gpu(fn, steps, warmup, stream):
    """Wall seconds per step (synchronised on both sides of the timed steps)
    and the per-launch durations from HIP events recorded on the launch
    stream between consecutive launches."""
    import torch
    warm_up(fn, warmup)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(steps)]
    return wall / steps, ev[0].elapsed_time(ev[steps]) * 1e-3 / steps, per


def time_gpu_graph(fn, steps, warmup, stream):
    """As time_gpu, with the timed steps replayed from a HIP graph: a batch
    of G calls (the largest G <= 25 dividing steps) is captured once and
    replayed steps/G times, so the host never paces short kernels.  Events
    bracket every replay; per-launch durations are a replay's time / G."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    per_graph = next(g for g in range(min(25, steps), 0, -1) if steps % g == 0)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                fn()
    torch.cuda.current_stream().wait_stream(side)
    # The graph's first replay uploads it.  Then untimed replays until the
    # warm-up has lasted MIN_WARMUP_SECONDS, ending right before the timed
    # ones: the capture leaves the GPU idle for a moment, and a timed replay
    # straight after it would start at a lowered clock.
    t0 = time.perf_counter()
    replays = 0
    while True:
        graph.replay()
        replays += 1
        if replays % 4 == 0:  # keep the host at most a few replays ahead
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= MIN_WARMUP_SECONDS:
                break
    torch.cuda.synchronize()
    WARMUP_RUN["launches"] = warmup + replays * per_graph
    reps = steps // per_graph
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(reps):
        graph.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e-3 / per_graph for i in range(reps)]
    return wall / steps, ev[0].elapsed_time(ev[reps]) * 1e-3 / steps, per


# the timer of the warm steps: graph replay (default) or eager launches
TIMER = {"fn": time_gpu_graph, "method": "HIP graph replays of a captured batch of calls"}


def time_cold(fn, launches, stream, scratch_mib=512):
    """Per-launch kernel durations with the caches flushed before each launch:
    a 512 MiB scratch buffer (twice the 256 MB MALL) is rewritten between
    launches, outside the timed events."""
    import torch
    scratch = torch.empty(scratch_mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda:0")
    per = []
    for i in range(launches):
        scratch.fill_(float(i))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        per.append(e0.elapsed_time(e1) * 1e-3)
    del scratch
    return per


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def _find_gfx_clock(node):
    """The shader (GFX) clock in MHz from amd-smi's JSON: the mean over the
    entries whose key names gfx (one per XCD) and whose 'clk' is a number or
    a {'value': number} dict, taken in the first dict that has any."""
    if isinstance(node, dict):
        vals = []
        for key, val in node.items():
            if "gfx" in str(key).lower() and isinstance(val, dict) and "clk" in val:
                clk = val["clk"]
                clk = clk.get("value") if isinstance(clk, dict) else clk
                try:
                    vals.append(float(clk))
                except (TypeError, ValueError):
                    pass
        if vals:
            return sum(vals) / len(vals)
        for val in node.values():
            found = _find_gfx_clock(val)
            if found is not None:
                return found
    elif isinstance(node, list):
        for val in node:
            found = _find_gfx_clock(val)
            if found is not None:
                return found
    return None


class ClockSampler:
    """Samples the GPU shader clock with amd-smi in a background thread while
    the GPU is kept busy.  Reports None when amd-smi or its output is not
    usable; the clock is context, not part of the result."""

    def __init__(self):
        import threading
        self.samples, self.error = [], None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _query(self):
        import subprocess
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"],
                             capture_output=True, text=True, timeout=20).stdout
        val = _find_gfx_clock(json.loads(out))
        if val is None:
            raise ValueError("no gfx clock in amd-smi output: " + out[:300])
        return val

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._query())
            except Exception as e:  # noqa: BLE001
                self.error = repr(e)[:400]
                return

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=30)

    def summary(self):
        if not self.samples:
            return {"gfx_mhz_median": None, "samples": 0, "source": "amd-smi", "error": self.error}
        return {"gfx_mhz_median": median(self.samples), "gfx_mhz_min": min(self.samples),
                "gfx_mhz_max": max(self.samples), "samples": len(self.samples), "source": "amd-smi",
                "window": "sampled while the same launches ran back to back for about 4 s"}


def cpu_baseline(w, q, k, v, seconds, o_gpu=None, lse_gpu=None):
    """The fp64 oracle, as it stands, on a time-boxed sample of the same
    workload: the first query rows of head 0, 1, ... against all N keys, with
    the BLAS thread pool set to every usable core.  When the GPU's O and LSE
    (host tensors of the timed launch) are given, the oracle rows it computed
    are also compared with them."""
    import numpy as np
    from oracle import attention
    from workloads import to_f64
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # noqa: BLE001
        limiter = None
    chunk = 256
    rows_done, t0 = 0, time.perf_counter()
    done = []  # (b, h, rows, o_ref, lse_ref)
    try:
        for b in range(w.B):
            for h in range(w.H):
                qf, kf, vf = (to_f64(t[b:b + 1, h:h + 1]) for t in (q, k, v))
                for r0 in range(0, w.N, chunk):
                    rows = np.arange(r0, min(r0 + chunk, w.N))
                    o_r, l_r = attention(qf, kf, vf, w.scale, causal=w.causal, rows=rows)
                    done.append((b, h, rows, o_r[0, 0], l_r[0, 0]))
                    rows_done += len(rows)
                    if time.perf_counter() - t0 >= seconds:
                        break
                if time.perf_counter() - t0 >= seconds:
                    break
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    finally:
        if limiter is not None:
            limiter.unregister()
    if w.causal:
        pairs = sum(float((rows + 1).sum()) for _, _, rows, _, _ in done)
    else:
        pairs = float(rows_done) * w.N
    flops = pairs * w.d * 4.0
    out = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle on {rows_done} query rows x {w.N} keys of {w.name} "
                   f"({rows_done / (w.B * w.H * w.N):.2%} of the workload), {dt:.1f} s wall; "
                   f"matmuls on {cores} BLAS threads (set explicitly), exp single-threaded"),
    }
    if o_gpu is not None:
        og, lg = to_f64(o_gpu), to_f64(lse_gpu)
        dmax = dsum = dl = num = den = 0.0
        cnt = 0
        for b, h, rows, o_r, l_r in done:
            d = np.abs(og[b, h, rows] - o_r)
            dmax = max(dmax, float(d.max()))
            dsum += float(d.sum())
            cnt += d.size
            dl = max(dl, float(np.abs(lg[b, h, rows] - l_r).max()))
            num += float(((og[b, h, rows] - o_r) ** 2).sum())
            den += float((o_r ** 2).sum())
        out["error_vs_oracle"] = {
            "rows": rows_done, "o_max_abs": dmax, "o_mean_abs": dsum / max(cnt, 1),
            "lse_max_abs": dl, "o_rel_fro": (num / den) ** 0.5 if den > 0 else 0.0,
            "bars": "bf16: max 2e-2, mean 2e-3, LSE 1e-3 (relative Frobenius checked at 1e-2 in the tests)",
            "of": "the O and LSE of the last timed launch, on the rows the oracle computed"}
    return out


def sparse_flops(w, m):
    """Algorithmic flops of a block-sparse call: 4*d per (query, key) pair of
    every set (128-row, 64-key) block, clipped at N; when causal, only the
    pairs with key <= query."""
    import numpy as np
    N = w.N
    i = np.arange(N)
    k0 = 64 * np.arange(m.shape[1])
    k1 = np.minimum(k0 + 64, N)
    lim = (i + 1)[:, None] if w.causal else N
    seen = np.clip(np.minimum(lim, k1[None, :]) - k0[None, :], 0, None)  # [N, key blocks]
    pairs = float((seen * np.asarray(m, dtype=bool)[i // 128]).sum())
    return 4.0 * w.B * w.H * pairs * w.d


def bench_one(w, steps, warmup, with_cpu, cpu_seconds, cold_launches=0, clock=False, mask="none",
              layout="contiguous", block_density=None, split=True):
    import torch
    import exact_attention_29_amd as ea
    from workloads import make_inputs

    dev = "cuda:0"
    q, k, v = make_inputs(w)
    B, H, N, d = w.shape
    if layout == "packed":
        # the same values in one [B, N, 3*H*d] input-projection output, read
        # in place through head views (attn_fwd_strided)
        x = torch.empty(B, N, 3 * H * d, dtype=q.dtype, device=dev)
        qd, kd, vd = (t.view(B, N, H, d).transpose(1, 2) for t in x.chunk(3, dim=-1))
        for dst, src in ((qd, q), (kd, k), (vd, v)):
            dst.copy_(src.to(dev))
    else:
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # key padding as the pages' layer passes it: every key valid (an all-False
    # padding mask), given as a per-entry length or as a byte mask
    masks = {"split": split}
    if mask == "len":
        masks["key_len"] = torch.full((B,), N, dtype=torch.int32, device=dev)
    elif mask == "bytes":
        # packed once, outside the timed calls (attn_pack_key_mask)
        masks["key_bits"] = ea.pack_key_mask(torch.ones((B, N), dtype=torch.bool, device=dev))
    flops = w.flops
    if block_density is not None:
        # a random block pattern with this fraction of (128-row, 64-key) blocks
        # set; flops count only the set blocks
        import numpy as np
        rng = np.random.default_rng(1000)
        m = rng.random((-(-N // 128), -(-N // 64))) < block_density
        masks["block_mask"] = torch.from_numpy(m).to(dev)
        flops = sparse_flops(w, m)

    # workspace: device memory a call needs beyond its outputs.  O and LSE
    # are allocated first (the allocator rounds blocks, so their own sizes
    # are not subtracted afterwards); then the call's peak allocation above
    # the level before it and the change of free device memory are read.
    out_bytes = o.numel() * o.element_size() + lse.numel() * 4
    # one call first: the first launch makes the runtime load the code object
    ea.forward(qd, kd, vd, scale=w.scale, causal=w.causal, out=o, lse=lse, **masks)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    free0 = torch.cuda.mem_get_info(dev)[0]
    ea.forward(qd, kd, vd, scale=w.scale, causal=w.causal, out=o, lse=lse, **masks)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated(dev) - base
    free_delta = free0 - torch.cuda.mem_get_info(dev)[0]

    def step():
        ea.forward(qd, kd, vd, scale=w.scale, causal=w.causal, out=o, lse=lse, **masks)

    wall, kern, per = TIMER["fn"](step, steps, warmup, stream)
    warm_run = WARMUP_RUN["launches"]
    if block_density is not None:
        # the same call without the block mask, for the time ratio
        dense_masks = {kk: vv for kk, vv in masks.items() if kk != "block_mask"}
        dense_masks["split"] = False  # the kernel the block-sparse one mirrors
        _, dense_kern, _ = TIMER["fn"](lambda: ea.forward(qd, kd, vd, scale=w.scale, causal=w.causal, out=o,
                                                       lse=lse, **dense_masks), steps, warmup, stream)
    clock_info = None
    if clock:
        # amd-smi takes about a second per query: keep the GPU busy with the
        # same launches for ~4 s while a thread samples it
        with ClockSampler() as clk:
            for _ in range(max(1, int(4.0 / kern))):
                step()
            torch.cuda.synchronize()
        clock_info = clk.summary()
    value = flops / wall / 1e12
    achieved = flops / kern / 1e12
    traffic = traffic_for(w.name)
    alg_bytes = 4 * B * H * N * d * 2 + 4 * B * H * N
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
            "block_sparse": None if block_density is None else {
                "density_target": block_density, "blocks_set": int(masks["block_mask"].sum()),
                "blocks": int(masks["block_mask"].numel()), "block": "128 queries x 64 keys",
                "flops_counted": "set blocks only",
                "time_vs_dense": round(kern / dense_kern, 4)},
            "layout": {"contiguous": "[B,H,N,d] contiguous",
                       "packed": "head views of one packed [B,N,3*H*d] projection (attn_fwd_strided)"}[layout],
            "key_mask": {"none": "none", "len": "key_len = N per entry (attn_fwd_masked)",
                         "bytes": "key mask all true, packed to bits (attn_fwd_masked, mask path)"}[mask],
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
            "kernel": kernel_name(w, B, H, N, block_density is not None, mask == "bytes", split),
            "kernel_ms": round(kern * 1e3, 4),
            "algorithmic_bytes": alg_bytes,
            # at the ridge (short sequences) the HBM view matters as well
            "hbm_view": {"achieved": round(alg_bytes / kern / 1e9, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s (algorithmic bytes / kernel time)",
                         "frac": round(alg_bytes / kern / 1e9 / PEAK_HBM_GBS, 4)},
        },
        "workspace": {"extra_bytes": int(extra), "mem_get_info_delta": int(free_delta),
                      "output_bytes": int(out_bytes),
                      "split_workspace_bytes": int(ea.attn_fwd_split_workspace_size(B, H, N, w.causal))
                      if split and not w.causal and block_density is None else 0,
                      "note": "extra: per call, beyond O and LSE; split_workspace_bytes: what this call "
                              "needs for attn_fwd_split (0: not split), held once per device and stream by "
                              "forward(), the same for every split call"},
        "warmup_launches_run": warm_run,
        "timing": {"kernel_ms_mean": round(kern * 1e3, 4), "kernel_ms_median": round(median(per) * 1e3, 4),
                   "kernel_ms_min": round(min(per) * 1e3, 4), "launches": steps,
                   "tflops_at_median": round(flops / median(per) / 1e12, 2),
                   "method": TIMER["method"],
                   "cache": "warm: inputs stay resident in L2/MALL between launches"},
    }
    if clock_info is not None:
        line["clock"] = clock_info
        mhz = clock_info.get("gfx_mhz_median")
        if mhz:
            peak_at_clock = PEAK_BF16_TFLOPS * mhz / 2400.0
            line["clock"]["bf16_peak_at_clock"] = round(peak_at_clock, 1)
            line["clock"]["pct_of_peak_at_clock"] = round(100.0 * achieved / peak_at_clock, 2)
    if cold_launches:
        cper = time_cold(step, cold_launches, stream)
        line["cold"] = {"kernel_ms_median": round(median(cper) * 1e3, 4),
                        "kernel_ms_min": round(min(cper) * 1e3, 4), "launches": cold_launches,
                        "tflops_at_median": round(flops / median(cper) / 1e12, 2),
                        "cache": "cold: a 512 MiB buffer is rewritten before every launch"}
    if with_cpu:
        log("[bench] timing the fp64 oracle on a sample ...")
        # o and lse still hold the last timed launch's output
        o_host, lse_host = o.cpu(), lse.cpu()
        cb = cpu_baseline(w, q, k, v, cpu_seconds, o_host, lse_host)
        err = cb.pop("error_vs_oracle", None)
        line["cpu_baseline"] = cb
        if err is not None:
            line["error_vs_oracle"] = err
    return line


def bench_backward(w, steps, warmup, key_len=None, key_density=None, block_density=None, layout="contiguous"):
    """attn_bwd (two kernels: dQ with the per-row terms, then dK/dV) on the workload, inputs and
    the forward's O, LSE resident.  FLOPs: the algorithmic 10*B*H*N^2*d of
    the recomputing backward pass (recompute S, then dV, dP, dQ, dK: five
    N x N x d products), halved when causal; this implementation recomputes S
    and dP in both the key-parallel and the query-parallel kernel (14*N^2*d
    executed).  key_len: every entry keeps this many valid keys; key_density:
    a random key bit mask (seed 1001) keeps about this fraction of each
    entry's keys (attn_bwd_masked, after the forward with the same masks);
    FLOPs then count the visible (query, key) pairs only: 10*d per pair.
    block_density: a random block mask as in the forward's block-sparse
    lines (seed 1000; attn_bwd_block_sparse), FLOPs over the visible pairs
    of the set blocks.  layout "packed": q, k, v head views of one packed
    [B, N, 3*H*d] projection, dO and O token-major [B, N, H, d], and dq,
    dk, dv written into head views of one packed gradient buffer
    (attn_bwd_strided)."""
    import numpy as np
    import torch
    import exact_attention_29_amd as ea
    from workloads import make_inputs, Workload

    dev = "cuda:0"
    B, H, N, d = w.shape
    q, k, v = (t.to(dev) for t in make_inputs(w))
    do = make_inputs(Workload("do", B, H, N, d, "bf16", 1.0, w.scale, w.causal, w.seed + 50, ""))[0].to(dev)
    if layout == "packed":
        if block_density is not None:
            raise SystemExit("--layout packed takes no --block-density")
        x = torch.empty(B, N, 3 * H * d, dtype=q.dtype, device=dev)
        views = [t.view(B, N, H, d).transpose(1, 2) for t in x.chunk(3, dim=-1)]
        for dst, src in zip(views, (q, k, v)):
            dst.copy_(src)
        q, k, v = views
        do_tok = torch.empty(B, N, H, d, dtype=q.dtype, device=dev)
        do_tok.transpose(1, 2).copy_(do)
        do = do_tok.transpose(1, 2)
    kl = None if key_len is None else torch.full((B,), key_len, dtype=torch.int32, device=dev)
    kvalid = None
    if key_density is not None:
        kvalid = np.random.default_rng(1001).random((B, N)) < key_density
        if key_len is not None:
            kvalid &= np.arange(N)[None, :] < key_len
    kbits = None if kvalid is None else ea.pack_key_mask(torch.tensor(kvalid, device=dev))
    bmask = None
    if block_density is not None:
        bm_np = np.random.default_rng(1000).random((-(-N // 128), -(-N // 64))) < block_density
        bmask = torch.from_numpy(bm_np).to(dev)
    o_tok = torch.empty(B, N, H, d, dtype=q.dtype, device=dev) if layout == "packed" else None
    o, lse = ea.forward(q, k, v, scale=w.scale, causal=w.causal, key_len=kl, key_bits=kbits, block_mask=bmask,
                        out=None if o_tok is None else o_tok.transpose(1, 2))
    if layout == "packed":
        gx = torch.empty(B, N, 3 * H * d, dtype=q.dtype, device=dev)
        dq, dk, dv = (t.view(B, N, H, d).transpose(1, 2) for t in gx.chunk(3, dim=-1))
        layouts = [ea._layout(t) for t in (q, k, v, o, do, dq, dk, dv)]
    else:
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(ea.attn_bwd_workspace_size(B, H, N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr())

    def step():
        # the current stream at call time (a capture stream while recording a graph)
        s = torch.cuda.current_stream(dev).cuda_stream
        if bmask is not None:
            ea.attn_bwd_block_sparse(*ptrs, B, H, N, d, w.scale, w.causal, bmask.data_ptr(), s)
        elif layout == "packed":
            ea.attn_bwd_strided(*ptrs, B, H, N, d, w.scale, w.causal, layouts, 0 if kl is None else kl.data_ptr(),
                                0 if kbits is None else kbits.data_ptr(), s)
        elif kl is None and kbits is None:
            ea.attn_bwd(*ptrs, B, H, N, d, w.scale, w.causal, s)
        else:
            ea.attn_bwd_masked(*ptrs, B, H, N, d, w.scale, w.causal, 0 if kl is None else kl.data_ptr(),
                               0 if kbits is None else kbits.data_ptr(), s)

    wall, kern, per = TIMER["fn"](step, steps, warmup, stream)
    warm_run = WARMUP_RUN["launches"]
    if bmask is not None:
        flops = 2.5 * sparse_flops(w, bm_np)
        counted = (f"10*d per visible (query, key) pair of the set blocks ({int(bm_np.sum())} of {bm_np.size})"
                   + (", key <= query" if w.causal else ""))
    elif kl is None and kvalid is None:
        flops = 10.0 * B * H * N * N * d * (0.5 if w.causal else 1.0)
        counted = "10*B*H*N^2*d (x0.5 causal)"
    elif kvalid is None:
        lk = max(0, min(key_len, N))
        pairs = sum(min(i + 1, lk) for i in range(N)) if w.causal else N * lk
        flops = 10.0 * B * H * pairs * d
        counted = f"10*d per visible (query, key) pair: {pairs} pairs per head (key_len {lk})"
    else:
        # visible pairs per entry: row i sees the valid keys j (j <= i when causal)
        per_entry = [int(np.cumsum(kv).sum()) if w.causal else int(kv.sum()) * N for kv in kvalid]
        pairs = sum(per_entry)
        flops = 10.0 * H * pairs * d
        counted = f"10*d per visible (query, key) pair: {pairs} pairs over the {B} entries (key density {key_density})"
    return {
        "metric": "attention backward (dQ, dK, dV) TFLOP/s",
        "value": round(flops / wall / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.what}", "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "scale": w.scale, "key_len": key_len, "key_density": key_density,
                   "block_density": block_density, "layout": layout, "flops_counted": counted},
        "pct_of_bf16_peak": round(100.0 * flops / wall / 1e12 / PEAK_BF16_TFLOPS, 2),
        "warmup_launches_run": warm_run,
        "timing": {"ms_mean": round(kern * 1e3, 4), "ms_median": round(median(per) * 1e3, 4),
                   "ms_min": round(min(per) * 1e3, 4),
                   "method": TIMER["method"],
                   "note": "the two kernels of one call, between events on the launch stream"},
        "workspace": {"bytes": int(ws.numel()),
                      "note": "caller-owned attn_bwd_workspace_size(B, H, N): LSE*log2(e) and -D per padded row"},
    }


def workspace_sweep():
    """Device memory one call needs beyond its outputs, over the patch counts
    of the 0.5-8 MP workloads, with the two fits: extra = c*P + d and
    extra = a*P^2 + b*P (a materialised score table would give a = 2*H
    bytes per P^2 for bf16)."""
    import numpy as np
    import torch
    import exact_attention_29_amd as ea
    from workloads import PATCH_SWEEP, WORKLOADS, make_inputs

    dev = "cuda:0"
    rows = []
    for n in list(PATCH_SWEEP) + [WORKLOADS["patch_3mp"].N, WORKLOADS["patch_8mp"].N]:
        w = WORKLOADS["patch_3mp"].with_n(n)
        q, k, v = (t.to(dev) for t in make_inputs(w))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, n), dtype=torch.float32, device=dev)
        out_bytes = o.numel() * o.element_size() + lse.numel() * 4
        # one call first: the first launch makes the runtime load the code object
        ea.forward(q, k, v, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        free0 = torch.cuda.mem_get_info(dev)[0]
        ea.forward(q, k, v, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        peak_extra = torch.cuda.max_memory_allocated(dev) - base
        free_delta = free0 - torch.cuda.mem_get_info(dev)[0]
        rows.append({"P": n, "extra_bytes": int(peak_extra), "output_bytes": int(out_bytes),
                     "mem_get_info_delta": int(free_delta),
                     "score_table_bytes_avoided": int(w.B * w.H * n * n * 2)})
        log(f"[workspace] P={n}: extra {peak_extra} B beyond {out_bytes} B of outputs")
        del q, k, v, o, lse
    P = np.array([r["P"] for r in rows], dtype=np.float64)
    E = np.array([r["extra_bytes"] for r in rows], dtype=np.float64)
    lin = np.linalg.lstsq(np.stack([P, np.ones_like(P)], 1), E, rcond=None)[0]
    quad = np.linalg.lstsq(np.stack([P * P, P], 1), E, rcond=None)[0]
    return {"workspace_sweep": rows,
            "fit_linear": {"c_bytes_per_P": float(lin[0]), "d_bytes": float(lin[1])},
            "fit_quadratic": {"a_bytes_per_P2": float(quad[0]), "b_bytes_per_P": float(quad[1])},
            "method": "O and LSE allocated first; then torch max_memory_allocated during the "
                      "call minus allocated before it, and the hipMemGetInfo free-memory delta"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU clock ramps for ~60 launches (~35 ms) from idle; 100 untimed
    # warmup steps put the timed steps in steady state.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="patch_3mp")
    ap.add_argument("--n", type=int, default=None, help="override the sequence length")
    ap.add_argument("--heads", type=int, default=None, help="override the head count")
    ap.add_argument("--causal", choices=["yes", "no"], default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--sweep", default=None, help="write one JSON line per workload to this file")
    ap.add_argument("--cold", type=int, default=30,
                    help="launches timed with flushed caches after the warm steps (0: skip)")
    ap.add_argument("--no-clock", action="store_true", help="do not sample the clock with amd-smi")
    ap.add_argument("--eager", action="store_true",
                    help="time the warm steps as eager launches from Python instead of HIP graph replays")
    ap.add_argument("--backward", action="store_true",
                    help="time attn_bwd (dQ, dK, dV) instead of the forward pass")
    ap.add_argument("--key-len", type=int, default=None,
                    help="with --backward: every batch entry has this many valid keys (attn_bwd_masked)")
    ap.add_argument("--key-density", type=float, default=None,
                    help="with --backward: a random key bit mask keeping this fraction of keys (attn_bwd_masked)")
    ap.add_argument("--block-density", type=float, default=None,
                    help="time attn_fwd_block_sparse with this fraction of random blocks set")
    ap.add_argument("--layout", choices=["contiguous", "packed"], default="contiguous",
                    help="read q, k, v as head views of one packed projection output")
    ap.add_argument("--mask", choices=["none", "len", "bytes"], default="none",
                    help="time attn_fwd_masked with every key valid, as a length or a byte mask")
    ap.add_argument("--no-split", action="store_true",
                    help="call forward(split=False): no key split of the last round (attn_fwd / attn_fwd_strided)")
    ap.add_argument("--workspace-sweep", action="store_true",
                    help="only measure the device memory a call needs beyond O and LSE, "
                         "at P = 1,944 .. 38,400, and fit it against P")
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

    if args.eager:
        TIMER.update(fn=time_gpu, method="eager launches from Python, events between launches")

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

    if args.backward:
        w = WORKLOADS[args.workload]
        if args.n:
            w = w.with_n(args.n)
        if args.causal:
            from dataclasses import replace
            w = replace(w, causal=args.causal == "yes")
        print(json.dumps(bench_backward(w, args.steps, args.warmup, args.key_len, args.key_density,
                                        args.block_density, args.layout)), flush=True)
        return

    if args.workspace_sweep:
        print(json.dumps(workspace_sweep()), flush=True)
        return

    if args.sweep:
        cases = [WORKLOADS[n] for n in ("bert_large", "gpt2_small_causal")]
        cases += [WORKLOADS["patch_3mp"].with_n(n) for n in PATCH_SWEEP]
        cases += [WORKLOADS["patch_3mp"], WORKLOADS["patch_8mp"]]
        from dataclasses import replace
        cases.append(replace(WORKLOADS["patch_3mp"], causal=True, name="patch_3mp_causal"))
        cases = [(c, "none", "contiguous", None) for c in cases]
        cases += [(WORKLOADS["patch_3mp"], "len", "contiguous", None),
                  (WORKLOADS["patch_3mp"], "bytes", "contiguous", None),
                  (WORKLOADS["bert_large"], "bytes", "contiguous", None),
                  (WORKLOADS["patch_3mp"], "none", "packed", None),
                  (WORKLOADS["patch_8mp"], "none", "packed", None),
                  (WORKLOADS["patch_3mp"], "none", "contiguous", 1.0),
                  (WORKLOADS["patch_3mp"], "none", "contiguous", 0.5),
                  (WORKLOADS["patch_3mp"], "none", "contiguous", 0.25),
                  (WORKLOADS["patch_8mp"], "none", "contiguous", 0.25)]
        with open(args.sweep, "w") as f:
            for w, mask, layout, dens in cases:
                steps = max(args.steps, 200) if w.flops < 2e10 else args.steps
                warm = max(args.warmup, 1000) if w.flops < 2e10 else args.warmup
                log(f"[bench] {w.name} {w.shape} causal={w.causal} mask={mask} layout={layout} density={dens}")
                line = bench_one(w, steps, warm, False, 0, mask=mask, layout=layout, block_density=dens,
                                 split=not args.no_split)
                f.write(json.dumps(line) + "\n")
                f.flush()
                log(f"[bench] {w.name}: {line['value']} TFLOP/s, kernel {line['roofline']['kernel_ms']} ms")
        return

    w = WORKLOADS[args.workload]
    if args.n:
        w = w.with_n(args.n)
    if args.heads:
        from dataclasses import replace
        w = replace(w, H=args.heads, name=f"{w.name}_h{args.heads}")
    if args.causal:
        from dataclasses import replace
        w = replace(w, causal=args.causal == "yes")
    log(f"[bench] {w.name} {w.shape} {w.dtype} causal={w.causal} steps={args.steps} warmup={args.warmup}")
    line = bench_one(w, args.steps, args.warmup, not args.no_cpu_baseline, args.cpu_seconds,
                     cold_launches=args.cold, clock=not args.no_clock, mask=args.mask,
                     layout=args.layout, block_density=args.block_density, split=not args.no_split)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
