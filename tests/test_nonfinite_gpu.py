"""Non-finite inputs on the GPU against the fp64 oracle.

The kernels do not scrub their inputs.  Under the definition (the oracle):
a NaN in a K row makes the score of every query that sees that key NaN, so
those rows are NaN in O and LSE, while rows that never see the key (causal
rows before it) are untouched; a NaN in feature f of a V row makes column f
of O NaN in every row that sees the key, and leaves the other features and
LSE alone.  The NaN positions must match the oracle's, and every finite
element must meet the usual bars.

One documented difference on the bf16 path: a wave multiplies a whole
32-key block of V by its probabilities, and a hidden key's probability is
an exact 0, so a NaN value of a hidden key reaches column f of the rows that
share its block (causal rows 32*floor(j/32) .. j-1 here).  The fp32 path
skips hidden keys and matches the oracle exactly.
"""

import numpy as np
import pytest
import torch

import exact_attention_29_amd as ea
from oracle import attention as oracle_attention
from tests.parity import BF16, FP32, assert_within, errors
from workloads import Workload, make_inputs, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N, F = 300, 5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load_library()
    yield
    torch.cuda.synchronize()


def _run(q, k, v, causal, dtype):
    o, lse = ea.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=0.125, causal=causal)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


def _finite_parts_agree(o, lse, o_ref, lse_ref, bar, what):
    ok_o = np.isfinite(o_ref)
    ok_l = np.isfinite(lse_ref)
    e = errors(np.where(ok_o, o, 0.0), np.where(ok_l, lse, 0.0),
               np.where(ok_o, o_ref, 0.0), np.where(ok_l, lse_ref, 0.0))
    assert_within(e, {kk: vv for kk, vv in bar.items() if kk != "o_mean"}, what)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("j", [100, 128, 299])
def test_nan_key_row(j, causal, dtype):
    w = Workload("nan_k", 1, 2, N, 64, dtype, 1.0, 0.125, causal, 900 + j, "")
    q, k, v = make_inputs(w)
    k[:, 1, j] = float("nan")  # head 1 only: head 0 stays finite everywhere
    print(f"[case] NaN in K row {j} of head 1, causal={causal}, {dtype}", flush=True)
    o, lse = _run(q, k, v, causal, dtype)
    with np.errstate(invalid="ignore"):
        o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), 0.125, causal=causal)
    assert np.array_equal(np.isnan(o), np.isnan(o_ref)), "NaN positions of O"
    assert np.array_equal(np.isnan(lse), np.isnan(lse_ref)), "NaN positions of LSE"
    assert np.isnan(lse_ref[0, 1, j:]).all() and np.isfinite(lse_ref[0, 1, :j if causal else 0]).all()
    _finite_parts_agree(o, lse, o_ref, lse_ref, FP32 if dtype == "fp32" else BF16, "finite rows")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("j", [100, 128, 299])
def test_nan_value(j, causal, dtype):
    w = Workload("nan_v", 1, 2, N, 64, dtype, 1.0, 0.125, causal, 950 + j, "")
    q, k, v = make_inputs(w)
    v[:, 1, j, F] = float("nan")
    print(f"[case] NaN in V[{j}, {F}] of head 1, causal={causal}, {dtype}", flush=True)
    o, lse = _run(q, k, v, causal, dtype)
    with np.errstate(invalid="ignore"):
        o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), 0.125, causal=causal)
    # the oracle: column F of the rows that see key j, nothing else
    first = j if causal else 0
    assert np.isnan(o_ref[0, 1, first:, F]).all() and np.isfinite(o_ref[0, 1, :first]).all()
    nan_gpu = np.isnan(o)
    expect = np.isnan(o_ref)
    if causal and dtype == "bf16":
        # rows of the 32-key block holding j, before j: column F may be NaN
        band = np.zeros_like(expect)
        band[0, 1, 32 * (j // 32):j, F] = True
        assert not (nan_gpu & ~(expect | band)).any(), "NaN outside the rows that share key j's block"
        assert (nan_gpu | ~expect).all(), "a row that sees the NaN value is finite"
        o = np.where(band, o_ref, o)
        nan_gpu = np.isnan(o)
    assert np.array_equal(nan_gpu, expect), "NaN positions of O"
    assert np.isfinite(lse).all(), "a NaN value must not reach LSE"
    _finite_parts_agree(o, lse, o_ref, lse_ref, FP32 if dtype == "fp32" else BF16, "finite elements")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_nan_query_row(dtype):
    """A NaN in one query row makes that row NaN and no other (the bf16
    path's exact-max fallback then recomputes that row's wave)."""
    w = Workload("nan_q", 1, 2, N, 64, dtype, 1.0, 0.125, False, 990, "")
    q, k, v = make_inputs(w)
    q[:, 0, 77, 3] = float("nan")
    o, lse = _run(q, k, v, False, dtype)
    with np.errstate(invalid="ignore"):
        o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), 0.125)
    assert np.array_equal(np.isnan(o), np.isnan(o_ref)) and np.isnan(o_ref[0, 0, 77]).all()
    assert np.array_equal(np.isnan(lse), np.isnan(lse_ref)) and np.isnan(lse[0, 0, 77])
    _finite_parts_agree(o, lse, o_ref, lse_ref, FP32 if dtype == "fp32" else BF16, "other rows")


def test_padded_nan_key_fp32_takes_no_part():
    """fp32 path: a key hidden by the padding mask with NaN in K and V leaves
    every row as if the key held finite values."""
    w = Workload("nan_pad", 2, 2, N, 64, "fp32", 1.0, 0.125, False, 991, "")
    q, k, v = make_inputs(w)
    valid = torch.ones(2, N, dtype=torch.bool)
    valid[1, 150] = False
    k[1, :, 150] = float("nan")
    v[1, :, 150] = float("nan")
    o, lse = ea.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=0.125, key_valid=valid.to(DEV))
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), 0.125, key_valid=valid.numpy())
    assert np.isfinite(o_ref).all()
    assert_within(errors(to_f64(o), to_f64(lse), o_ref, lse_ref), FP32, "padded NaN key")
