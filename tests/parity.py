"""Comparison helpers shared by the GPU parity tests and the smoke check.

Bars (from the stated tolerances for this operation):
  bf16 I/O, fp32 accumulation: max |O - O_ref| <= 2e-2 and mean <= 2e-3;
  fp32 path:                   max |O - O_ref| <= 1e-5;
  LSE (both paths):            max |LSE - LSE_ref| <= 1e-3.
The oracle sees the same rounded bf16 inputs, so input rounding is not
counted as error.  Beside the bars, the relative Frobenius error of O is
checked against 1e-2: at the large patch workloads |O| is small (~5e-3 rms)
and the absolute bars alone would accept a badly scaled output.  The LSE
bar is the sharp detector of coverage mistakes (a dropped or repeated key
tile moves LSE by ~ln((N+64)/N) > 1e-3 at every size tested).
"""

import numpy as np

BF16 = dict(o_max=2e-2, o_mean=2e-3, lse_max=1e-3, rel_fro=1e-2)
FP32 = dict(o_max=1e-5, o_mean=1e-5, lse_max=1e-3, rel_fro=1e-5)


def errors(o, lse, o_ref, lse_ref):
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    d = np.abs(o - o_ref)
    return dict(
        o_max=float(d.max()) if d.size else 0.0,
        o_mean=float(d.mean()) if d.size else 0.0,
        lse_max=float(np.abs(lse - lse_ref).max()) if lse.size else 0.0,
        rel_fro=float(np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-300)),
        finite=bool(np.all(np.isfinite(o)) and np.all(np.isfinite(lse))),
    )


def assert_within(err, bar, what=""):
    assert err["finite"], f"{what}: non-finite output"
    for key, lim in bar.items():
        assert err[key] <= lim, f"{what}: {key} = {err[key]:.3e} > {lim:.1e} ({err})"
