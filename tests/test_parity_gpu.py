"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every test here runs the production entry points (attn_fwd / attn_fwd_fp32
via the Python binding) on cuda:0 and compares element by element with the
oracle on the same seeded inputs: in full where the oracle finishes in
seconds (every row of the 0.5-3 MP patch workloads included), and at 8 MP on
eight random 256-row blocks per head (every row offset of a workgroup) plus
the last block.
"""

import math

import numpy as np
import pytest
import torch

import exact_attention_29_amd as ea
from oracle import attention as oracle_attention
from tests.parity import BF16, FP32, assert_within, bf16_ulp, errors
from workloads import PATCH_SWEEP, WORKLOADS, Workload, block_rows, make_inputs, sample_rows, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load_library()
    yield
    torch.cuda.synchronize()


def gpu_run(q, k, v, scale, causal):
    o, lse = ea.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


def compare(w, q, k, v, o, lse, rows=None, what=""):
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    o_ref, lse_ref = oracle_attention(qf, kf, vf, w.scale, causal=w.causal, rows=rows)
    o_h, lse_h = to_f64(o), to_f64(lse)
    if rows is not None:
        o_h, lse_h = o_h[:, :, rows], lse_h[:, :, rows]
    err = errors(o_h, lse_h, o_ref, lse_ref)
    assert_within(err, FP32 if w.dtype == "fp32" else BF16, what or w.name)
    return err


def bf16_workload(n, causal, B=2, H=3, seed=100, sigma=1.0, scale=0.125):
    return Workload(f"edge_N{n}_{'c' if causal else 'nc'}", B, H, n, 64, "bf16", sigma, scale,
                    causal, seed + n, "edge size")


# ------------------------------------------------------------ the workloads

@pytest.mark.parametrize("name", ["tiny", "bert_large", "gpt2_small_causal"])
def test_workload_full(name):
    w = WORKLOADS[name]
    print(f"[case] {name} {w.shape} {w.dtype} causal={w.causal}", flush=True)
    q, k, v = make_inputs(w)
    o, lse = gpu_run(q, k, v, w.scale, w.causal)
    err = compare(w, q, k, v, o, lse)
    print(f"[ok] {name} {err}", flush=True)


@pytest.mark.parametrize("n", list(PATCH_SWEEP) + [11616])
def test_patch_workload_full(n):
    """The 0.5-3 MP patch workloads, every row of every head."""
    w = WORKLOADS["patch_3mp"] if n == 11616 else WORKLOADS["patch_3mp"].with_n(n)
    print(f"[case] {w.name} {w.shape} all rows", flush=True)
    q, k, v = make_inputs(w)
    o, lse = gpu_run(q, k, v, w.scale, w.causal)
    err = compare(w, q, k, v, o, lse)
    print(f"[ok] {w.name} {err}", flush=True)


def test_patch_8mp_blocks():
    """8 MP (P = 38,400): per head, eight random 256-row blocks (every row
    offset of an 8-wave workgroup) plus the last block, 2,048-2,304 rows a
    head."""
    w = WORKLOADS["patch_8mp"]
    print(f"[case] {w.name} {w.shape}", flush=True)
    q, k, v = make_inputs(w)
    o, lse = gpu_run(q, k, v, w.scale, w.causal)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    o_h, lse_h = to_f64(o), to_f64(lse)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for h in range(w.H):
        rows = block_rows(w.N, 8, seed=4000 + h)
        ro, rl = oracle_attention(qf[:, h:h + 1], kf[:, h:h + 1], vf[:, h:h + 1], w.scale, rows=rows)
        ref_o.append(ro)
        ref_l.append(rl)
        got_o.append(o_h[:, h:h + 1, rows])
        got_l.append(lse_h[:, h:h + 1, rows])
    # heads may differ in row count (a random block can be the last one)
    err = errors(np.concatenate(got_o, 2), np.concatenate(got_l, 2), np.concatenate(ref_o, 2),
                 np.concatenate(ref_l, 2))
    assert_within(err, BF16, w.name)
    print(f"[ok] {w.name} rows={sum(r.shape[2] for r in ref_o)} {err}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_patch_3mp_causal_variant(causal):
    """The 3 MP shape also run causal (the causal skip at 182 tiles), every row."""
    w = Workload("patch_3mp_causal", 1, 16, 11616, 64, "bf16", 0.5, 0.125, causal, 3, "")
    q, k, v = make_inputs(w)
    o, lse = gpu_run(q, k, v, w.scale, w.causal)
    compare(w, q, k, v, o, lse)


@pytest.mark.parametrize("B, H", [(3, 21), (4, 16)])
def test_wave_count_threshold(B, H):
    """Non-causal calls take 8-wave workgroups (256 rows) when those give
    each of the 256 CUs one, else 4-wave ones: at N = 1000 (4 row blocks of
    256), 63 heads take the 4-wave kernel and 64 heads the 8-wave one."""
    w = Workload(f"threshold_{B}x{H}", B, H, 1000, 64, "bf16", 1.0, 0.125, False, 4000 + H, "")
    q, k, v = make_inputs(w)
    o, lse = gpu_run(q, k, v, w.scale, False)
    compare(w, q, k, v, o, lse)


# ------------------------------------------------------------ edge sizes

EDGE_N = [1, 2, 3, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 511, 513, 1000]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", EDGE_N)
def test_edge_sizes_bf16(n, causal):
    w = bf16_workload(n, causal)
    print(f"[case] bf16 N={n} causal={causal}", flush=True)
    q, k, v = make_inputs(w)
    o, lse = gpu_run(q, k, v, w.scale, causal)
    compare(w, q, k, v, o, lse)


# Key-tile counts 1 .. 21 with whole, one-half (32 keys) and ragged last
# tiles: every length of the last, partial turn of the LDS ring (6 stages
# without a mask, 5 causal), barriers after tiles of either parity, and the
# tail after each (a drain of one or two half tiles when the last tile needs
# no mask, the general path otherwise).
RING_N = [64 * t + r for t in range(1, 21) for r in (0, 37)] + [64 * t + 32 for t in range(1, 21, 2)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", RING_N)
def test_ring_lengths_bf16(n, causal):
    w = bf16_workload(n, causal, B=1, H=2, seed=5000 + n)
    print(f"[case] ring bf16 N={n} causal={causal}", flush=True)
    q, k, v = make_inputs(w)
    o, lse = gpu_run(q, k, v, w.scale, causal)
    compare(w, q, k, v, o, lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 63, 64, 65, 100, 128, 129, 257])
def test_edge_sizes_fp32(n, causal):
    w = Workload(f"fp32_N{n}", 2, 2, n, 64, "fp32", 1.0, 0.125, causal, 200 + n, "")
    print(f"[case] fp32 N={n} causal={causal}", flush=True)
    q, k, v = make_inputs(w)
    o, lse = gpu_run(q, k, v, w.scale, causal)
    compare(w, q, k, v, o, lse)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 1.0, 0.01])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_other_scales(scale, dtype):
    """Negative, zero, large and small scales, at the stated bars (the fp32
    path forms scores in fp64, so 1e-5 holds at scale 1 too)."""
    for causal in (False, True):
        w = Workload("scale", 1, 2, 200, 64, dtype, 1.0, scale, causal, 300, "")
        q, k, v = make_inputs(w)
        o, lse = gpu_run(q, k, v, scale, causal)
        compare(w, q, k, v, o, lse, what=f"scale={scale} {dtype} causal={causal}")


# ------------------------------------------------------------ invariants

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [200, 3952])
def test_constant_values_give_constant_output(n, causal):
    """V = c (a bf16 value): every output element is exactly c after rounding."""
    w = bf16_workload(n, causal, B=1, H=4)
    q, k, _ = make_inputs(w)
    for c in (0.375, -1.25):
        v = torch.full_like(q, c)
        o, _ = gpu_run(q, k, v, w.scale, causal)
        assert bool((o.float() == c).all()), f"constant V={c}: {o.float().unique()[:8]}"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_single_key_gives_values(dtype):
    w = Workload("n1", 3, 5, 1, 64, dtype, 1.0, 0.125, False, 400, "")
    q, k, v = make_inputs(w)
    for causal in (False, True):
        o, lse = gpu_run(q, k, v, w.scale, causal)
        assert torch.equal(o.cpu(), v), "N=1: O != V"
        ref = w.scale * (to_f64(q) * to_f64(k)).sum(-1)
        assert np.abs(to_f64(lse) - ref).max() <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_causal_row_zero_is_v0(dtype):
    w = Workload("row0", 2, 3, 777, 64, dtype, 1.0, 0.125, True, 401, "")
    q, k, v = make_inputs(w)
    o, _ = gpu_run(q, k, v, w.scale, True)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


def test_key_value_permutation():
    w = bf16_workload(1000, False, B=1, H=2)
    q, k, v = make_inputs(w)
    perm = torch.from_numpy(np.random.default_rng(7).permutation(w.N))
    o1, l1 = gpu_run(q, k, v, w.scale, False)
    o2, l2 = gpu_run(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), w.scale, False)
    a, b = to_f64(o1), to_f64(o2)
    # Permuting keys changes the order of the key tiles, hence the running max
    # against which each probability is formed and rounded to bf16.  Each
    # rounded probability is within 2^-8 (relative) of its exact value, so
    # each result is within 2^-8 * sum_j p_j |v_j| of the exact-probability
    # result (plus output rounding and fp32 noise), and the two results within
    # twice that.  sum_j p_j |v_j| is the oracle's output for |V|.
    w_abs, _ = oracle_attention(to_f64(q), to_f64(k), np.abs(to_f64(v)), w.scale)
    tol = 2.0 ** -7 * w_abs + bf16_ulp(a) + bf16_ulp(b) + 1e-6
    bad = np.abs(a - b) > tol
    assert not bad.any(), f"{bad.sum()} elements differ; max {np.abs(a - b).max():.3e}"
    assert np.abs(to_f64(l1) - to_f64(l2)).max() <= 1e-5


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [129, 11616])
def test_uniform_attention_closed_form(n, causal):
    """Q = 0: O_i is the mean of the visible values and LSE_i = ln(#visible).
    A dropped or repeated key tile, or unmasked padding keys, moves LSE by more
    than the 1e-3 bar at every N here."""
    w = Workload("uniform", 1, 2, n, 64, "bf16", 0.5, 0.125, causal, 402, "")
    _, k, v = make_inputs(w)
    q = torch.zeros_like(k)
    o, lse = gpu_run(q, k, v, w.scale, causal)
    cnt = np.arange(1, n + 1, dtype=np.float64) if causal else np.full(n, float(n))
    assert np.abs(to_f64(lse) - np.log(cnt)).max() <= 1e-3
    vf = to_f64(v)
    mean = np.cumsum(vf, axis=2) / cnt[:, None] if causal else np.broadcast_to(vf.mean(2, keepdims=True), vf.shape)
    assert np.abs(to_f64(o) - mean).max() <= 2e-2


def test_identity_closed_form():
    """Q = K = alpha * I rows (N <= 64): s_ij = beta [i == j], so
    P_ij = (e^beta [i==j] + [i!=j]) / (e^beta + seen - 1) and
    LSE_i = ln(e^beta + seen - 1), seen = N (or i + 1 when causal).
    beta = 3 ln 2 makes every probability exact in bf16 (1 and 1/8); beta = 2
    makes 47 equal off-diagonal probabilities that all round the same way in
    bf16, which the fp32 row sum must not inherit."""
    n, alpha = 48, 4.0
    eye = torch.zeros(1, 1, n, 64)
    eye[0, 0, torch.arange(n), torch.arange(n)] = 1.0
    q = (alpha * eye).to(torch.bfloat16)
    v = eye.to(torch.bfloat16)
    for beta in (3 * math.log(2), 2.0):
        scale = beta / (alpha * alpha)
        for causal in (False, True):
            o, lse = gpu_run(q, q, v, scale, causal)
            seen = np.arange(1, n + 1) if causal else np.full(n, n)
            exact = np.log(math.exp(beta) + seen - 1)
            assert np.abs(to_f64(lse)[0, 0] - exact).max() <= 1e-5, (beta, causal)
            p_diag = math.exp(beta) / (math.exp(beta) + seen - 1)
            assert np.abs(to_f64(o)[0, 0, np.arange(n), np.arange(n)] - p_diag).max() <= 4e-3


def test_one_hot_limit():
    """One score ~200 log2-units above the rest: O_i = V_argmax exactly."""
    n = 300
    rng = np.random.default_rng(403)
    q = torch.zeros(1, 1, n, 64)
    k = torch.from_numpy(0.01 * rng.standard_normal((1, 1, n, 64)).astype(np.float32))
    q[0, 0, :, 0] = 16.0
    k[0, 0, 137, 0] = 8.0
    v = torch.from_numpy(rng.standard_normal((1, 1, n, 64)).astype(np.float32))
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    o, _ = gpu_run(q, k, v, 1.0, False)
    assert torch.equal(o[0, 0].cpu(), v[0, 0, 137].expand(n, 64))


def _growth_inputs(n, growth, reverse=False, peak_last=False, seed=500):
    """q_i = 16 e_0 for every row; k_j = (16 * j / n) e_0 * growth/256, so the
    scaled score of key j (scale 1) rises linearly from 0 to `growth` natural
    units across the keys (falls, when reversed).  Small random values in the
    other features keep rows distinct."""
    rng = np.random.default_rng(seed)
    q = 0.01 * rng.standard_normal((1, 2, n, 64)).astype(np.float32)
    k = 0.01 * rng.standard_normal((1, 2, n, 64)).astype(np.float32)
    v = rng.standard_normal((1, 2, n, 64)).astype(np.float32)
    q[..., 0] = 16.0
    ramp = np.arange(n, dtype=np.float32) / n * (growth / 16.0)
    k[..., 0] = ramp[::-1] if reverse else ramp
    if peak_last:
        k[..., n - 1, 0] = growth / 16.0 + 4.0
    return tuple(torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("growth, reverse, peak_last", [
    (12.0, False, False),    # the max rises ~17 log2 units: steady state keeps p <= 2^17
    (200.0, False, False),   # rises ~290 log2 units: the per-wave exact fallback
    (200.0, True, False),    # max in the first tile, falling scores
    (40.0, False, True),     # max in the ragged last tile
])
def test_score_growth_paths(growth, reverse, peak_last, causal):
    n = 2000  # 63 half tiles, ragged end, long steady state
    q, k, v = _growth_inputs(n, growth, reverse, peak_last)
    w = Workload("growth", 1, 2, n, 64, "bf16", 1.0, 1.0, causal, 0, "")
    o, lse = gpu_run(q, k, v, 1.0, causal)
    compare(w, q, k, v, o, lse, what=f"growth={growth} reverse={reverse} peak_last={peak_last}")


def test_deterministic_repeat():
    w = WORKLOADS["bert_large"]
    q, k, v = (t.to(DEV) for t in make_inputs(w))
    o1, l1 = ea.forward(q, k, v, scale=w.scale)
    o2, l2 = ea.forward(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------ memory behaviour

@pytest.mark.parametrize("n", list(PATCH_SWEEP) + [WORKLOADS["patch_3mp"].N, WORKLOADS["patch_8mp"].N])
def test_workspace_is_zero_across_patch_counts(n):
    """Device memory a call needs beyond O and LSE, over the patch counts of
    the 0.5-8 MP workloads: none (a score table would need 2*H*P^2 bytes,
    47 GB at P=38,400).  O and LSE are allocated first, so the allocator's
    rounding of their blocks does not enter the measurement."""
    w = WORKLOADS["patch_3mp"].with_n(n)
    q, k, v = (t.to(DEV) for t in make_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, n, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    free0 = torch.cuda.mem_get_info()[0]
    ea.forward(q, k, v, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() - base == 0
    assert torch.cuda.mem_get_info()[0] == free0
    # and the result is right on sampled rows
    rows = sample_rows(n, 64, seed=n)
    compare(w, q.cpu(), k.cpu(), v.cpu(), o, lse, rows=rows, what=f"P={n}")


def test_no_workspace_and_no_out_of_bounds_writes():
    """The call allocates nothing beyond O and LSE, and writes nothing outside
    them: O and LSE sit inside guard bands filled with a canary."""
    w = WORKLOADS["patch_3mp"].with_n(1944)
    q, k, v = (t.to(DEV) for t in make_inputs(w))
    B, H, N, d = w.shape
    guard = 4096
    o_buf = torch.full((guard + B * H * N * d + guard,), -7.0, dtype=torch.bfloat16, device=DEV)
    l_buf = torch.full((guard + B * H * N + guard,), -7.0, dtype=torch.float32, device=DEV)
    o = o_buf[guard:guard + B * H * N * d].view(B, H, N, d)
    lse = l_buf[guard:guard + B * H * N].view(B, H, N)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ea.forward(q, k, v, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() - base == 0
    assert torch.cuda.mem_get_info()[0] == free0
    for buf in (o_buf, l_buf):
        assert bool((buf[:guard] == -7.0).all()) and bool((buf[-guard:] == -7.0).all())
    assert bool(torch.isfinite(o.float()).all())


def test_runs_on_the_callers_stream():
    w = bf16_workload(700, True)
    q, k, v = make_inputs(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qd, kd, vd = (t.to(DEV, non_blocking=False) for t in (q, k, v))
        o, lse = ea.forward(qd, kd, vd, scale=w.scale, causal=True)
    s.synchronize()
    compare(w, q, k, v, o, lse)


def test_errors_leave_outputs_untouched():
    q = torch.randn(1, 2, 64, 32, device=DEV).to(torch.bfloat16)
    with pytest.raises(ea.AttnError) as e:
        ea.forward(q, q, q)
    assert e.value.code == ea.ATTN_E_INVALID
    q = torch.randn(1, 2, 64, 64, device=DEV).to(torch.bfloat16)
    o = torch.full_like(q, 3.0)
    lse = torch.full((1, 2, 64), 3.0, device=DEV)
    with pytest.raises(ea.AttnError):
        ea.attn_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    1, 2, 64, 64, float("nan"), 0, None)
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((lse == 3.0).all())


@pytest.mark.parametrize("shape", [(1, 2, 0, 64), (0, 2, 5, 64), (2, 0, 5, 64)])
def test_empty_inputs_give_empty_outputs(shape):
    """Shapes with nothing to compute return empty outputs of the right shape
    (the C entry points take B, H, N >= 1; the binding answers these itself)."""
    q = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    o, lse = ea.forward(q, q, q)
    assert o.shape == shape and lse.shape == shape[:3]
    dq, dk, dv = ea.backward(q, q, q, o, lse, q)
    assert dq.shape == dk.shape == dv.shape == shape
    with pytest.raises(ea.AttnError):
        bad = torch.empty(shape[:3] + (32,), dtype=torch.bfloat16, device=DEV)
        ea.forward(bad, bad, bad)
