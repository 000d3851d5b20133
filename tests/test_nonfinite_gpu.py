"""Non-finite inputs on the GPU against the fp64 oracle.

The kernels do not scrub their inputs.  Under the definition (the oracle):
a NaN in a K row makes the score of every query that sees that key NaN, so
those rows are NaN in O and LSE, while rows that never see the key (causal
rows before it) are untouched; a NaN in feature f of a V row makes column f
of O NaN in every row that sees the key, and leaves the other features and
LSE alone.  An infinite K element gives a query +inf, -inf or NaN as
score by the sign of its matching Q feature: +inf makes the row NaN (the
max is +inf and exp(inf - inf) is NaN), -inf takes the key out; an infinite
V value makes that column of O infinite in the rows that see the key.  The
NaN and infinity positions must match the oracle's, and every finite element
must meet the usual bars.

One documented difference on the bf16 path: a wave multiplies a whole
32-key block of V by its probabilities, and a hidden key's probability is
an exact 0, so a non-finite value of a hidden key reaches column f of the
rows that share its block as NaN (0 * NaN, 0 * inf: causal rows
32*floor(j/32) .. j-1 here).  The key slots past N of a ragged length hold
copies of key N-1's V row, so a non-finite V[N-1] reaches every row that
visits that last block likewise (an infinite value gives NaN there, not
+-inf).  The fp32 path skips hidden keys and matches the oracle exactly.
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


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("j", [5, 128, 298])
def test_inf_key_element(j, causal, dtype):
    """K[j, F] = +inf: a query with q[F] > 0 scores +inf against key j (the
    definition's max is +inf and exp(inf - inf) is NaN: the row is NaN), one
    with q[F] < 0 scores -inf (key j takes no part: a finite row), and one
    with q[F] = 0 scores 0 * inf = NaN.  Key j sits in the first key tile,
    on a tile edge and in the ragged last tile, so both the exact first
    step and the steady state (with its exact-max fallback) meet it."""
    w = Workload("inf_k", 1, 2, N, 64, dtype, 1.0, 0.125, causal, 1010 + j, "")
    q, k, v = make_inputs(w)
    k[:, 1, j, F] = float("inf")
    mag = q[:, 1, :, F].abs() + 0.25
    rows = torch.arange(N)
    q[:, 1, :, F] = torch.where(rows % 3 == 0, torch.zeros_like(mag), torch.where(rows % 3 == 1, mag, -mag))
    print(f"[case] +inf in K[{j}, {F}] of head 1, causal={causal}, {dtype}", flush=True)
    o, lse = _run(q, k, v, causal, dtype)
    with np.errstate(invalid="ignore"):
        o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), 0.125, causal=causal)
    first = j if causal else 0
    sees = np.zeros(N, dtype=bool)
    sees[first:] = True
    r = np.arange(N)
    assert np.isnan(lse_ref[0, 1, sees & (r % 3 != 2)]).all(), "oracle: +inf or NaN score rows"
    assert np.isfinite(lse_ref[0, 1, ~sees | (r % 3 == 2)]).all(), "oracle: -inf score rows and rows before j"
    assert np.array_equal(np.isnan(o), np.isnan(o_ref)), "NaN positions of O"
    assert np.array_equal(np.isnan(lse), np.isnan(lse_ref)), "NaN positions of LSE"
    _finite_parts_agree(o, lse, o_ref, lse_ref, FP32 if dtype == "fp32" else BF16, "finite rows")


def _block_band(j, causal):
    """bf16 path: the (row, column F) elements of O that a non-finite V[j, F]
    may turn NaN beyond the definition -- rows that visit key j's 32-key
    block without seeing key j (causal rows 32*floor(j/32) .. j-1), and, for
    the last key of a ragged length, every row that visits that block: its
    key slots past N hold copies of key N-1's V row with probability 0."""
    band = np.zeros((1, 2, N, 64), dtype=bool)
    b0 = 32 * (j // 32)
    if causal:
        band[0, 1, b0:j, F] = True
    if j == N - 1 and N % 32:
        band[0, 1, b0 if causal else 0:, F] = True
    return band


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("j", [100, 298, 299])
def test_inf_value(j, causal, dtype):
    """V[j, F] = -inf: column F of O is -inf in every row that sees key j,
    nothing else changes.  On the bf16 path the elements of the 32-key block
    band may be NaN instead (0 * inf, as with a NaN value); key 299 is the
    last key of the ragged length 300."""
    w = Workload("inf_v", 1, 2, N, 64, dtype, 1.0, 0.125, causal, 1060 + j, "")
    q, k, v = make_inputs(w)
    v[:, 1, j, F] = float("-inf")
    print(f"[case] -inf in V[{j}, {F}] of head 1, causal={causal}, {dtype}", flush=True)
    o, lse = _run(q, k, v, causal, dtype)
    with np.errstate(invalid="ignore"):
        o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), 0.125, causal=causal)
    first = j if causal else 0
    assert np.isneginf(o_ref[0, 1, first:, F]).all() and np.isfinite(o_ref[0, 1, :first]).all()
    assert not np.isnan(o_ref).any()
    if dtype == "bf16":
        band = _block_band(j, causal)
        assert not np.isnan(np.where(band, 0.0, o)).any(), "NaN outside the band of key j's block"
        o = np.where(band & np.isnan(o), o_ref, o)
    assert np.array_equal(np.isneginf(o), np.isneginf(o_ref)), "-inf positions of O"
    assert not np.isnan(o).any() and np.isfinite(lse).all()
    _finite_parts_agree(o, lse, o_ref, lse_ref, FP32 if dtype == "fp32" else BF16, "finite elements")


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
