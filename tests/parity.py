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


def bf16_ulp(x):
    """The spacing of bf16 numbers at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def bf16_max_bound(o_ref, o_abs_ref, o_got):
    """Per-element max bar for rows far sharper than the workloads' (standard
    normal inputs with scales up to 1, not 1/8).  The probabilities that
    multiply V are rounded to bf16 (relative error at most 2^-8) while the row
    sum l adds the unrounded ones, so O_if moves by at most
    2^-8 * sum_j p_ij |v_jf| (o_abs_ref: the oracle's output for |V|); the
    final rounding of O adds half a bf16 ulp; 1e-6 covers the fp32 sums.
    Where that is below the fixed 2e-2 bar, the fixed bar holds."""
    ulp = bf16_ulp(np.maximum(np.abs(o_ref), np.abs(o_got)))
    return np.maximum(BF16["o_max"], 2.0 ** -8 * np.asarray(o_abs_ref) + 0.5 * ulp + 1e-6)


def assert_bf16_elementwise(o, lse, o_ref, lse_ref, o_abs_ref, what=""):
    """The bf16 bars with bf16_max_bound in place of the fixed max bar: mean,
    relative Frobenius and LSE bars unchanged."""
    o = np.asarray(o, dtype=np.float64)
    err = errors(o, lse, o_ref, lse_ref)
    assert_within(err, {key: lim for key, lim in BF16.items() if key != "o_max"}, what)
    bound = bf16_max_bound(o_ref, o_abs_ref, o)
    over = np.abs(o - o_ref) - bound
    assert not (over > 0).any(), (f"{what}: {(over > 0).sum()} elements above their bound; worst "
                                  f"|dO| = {np.abs(o - o_ref).flat[over.argmax()]:.3e} vs "
                                  f"{bound.flat[over.argmax()]:.3e} ({err})")


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


# Gradients (bf16 I/O): P and dS are rounded to bf16 before their products,
# O enters D = rowsum(dO * O) as bf16, and the results are rounded to bf16;
# each gradient stays within 1e-2 relative Frobenius error and within 2e-2
# of max|ref| at every element.  dS = P * (dP - D) cancels where the exact
# gradient is (nearly) zero, so the denominators are max(|ref|, 0.05 |mag|),
# mag being the same gradient with every cancelling difference replaced by
# its magnitude (grad_magnitudes).
GRAD = dict(rel_fro=1e-2, rel_max=2e-2)


def grad_magnitudes(q, k, v, do, scale, causal, key_valid=None):
    """The gradients with every cancelling difference replaced by its
    magnitude: dS -> P * (|dP| + |D|), dO -> |dO| (float64, from the oracle's
    own steps; key_valid: optional bool [B, N] key mask)."""
    from oracle import backward as ob
    from workloads import to_f64
    q, k, v, do = (to_f64(t) for t in (q, k, v, do))
    B, H, N, d = q.shape
    mq, mk, mv = (np.zeros((B, H, N, d)) for _ in range(3))
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            p = ob._probabilities(q[b, h], k[b, h], scale, causal, rows,
                                  None if key_valid is None else np.asarray(key_valid, dtype=bool)[b])
            dp = ob._dp(do[b, h], v[b, h])
            delta = ob._delta(p, dp)
            mds = p * (np.abs(dp) + np.abs(delta)[:, None])
            mq[b, h] = abs(scale) * (mds @ np.abs(k[b, h]))
            mk[b, h] = abs(scale) * (mds.T @ np.abs(q[b, h]))
            mv[b, h] = p.T @ np.abs(do[b, h])
    return mq, mk, mv


def grad_magnitudes_blocks(q, k, v, do, scale, causal, block_mask):
    """grad_magnitudes under a block mask (M, bq, bk)."""
    from oracle import backward as ob
    from workloads import to_f64
    q, k, v, do = (to_f64(t) for t in (q, k, v, do))
    B, H, N, d = q.shape
    mq, mk, mv = (np.zeros((B, H, N, d)) for _ in range(3))
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            p = ob._probabilities(q[b, h], k[b, h], scale, causal, rows, None, block_mask)
            dp = ob._dp(do[b, h], v[b, h])
            delta = ob._delta(p, dp)
            mds = p * (np.abs(dp) + np.abs(delta)[:, None])
            mq[b, h] = abs(scale) * (mds @ np.abs(k[b, h]))
            mk[b, h] = abs(scale) * (mds.T @ np.abs(q[b, h]))
            mv[b, h] = p.T @ np.abs(do[b, h])
    return mq, mk, mv


def assert_grad_within(name, got, ref, mag):
    from workloads import to_f64
    got = to_f64(got)
    err = got - ref
    fro = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 0.05 * np.linalg.norm(mag), 1e-300))
    mx = float(np.abs(err).max() / max(np.abs(ref).max(), 0.05 * np.abs(mag).max(), 1e-300))
    print(f"[bwd] {name}: rel_fro {fro:.2e}  max/maxref {mx:.2e}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    assert fro <= GRAD["rel_fro"], f"{name}: relative Frobenius error {fro:.3e} > {GRAD['rel_fro']}"
    assert mx <= GRAD["rel_max"], f"{name}: max error {mx:.3e} of max|ref| > {GRAD['rel_max']}"


def grad_magnitudes_sampled(q, k, v, do, scale, causal, rows, keys, key_valid=None, block_mask=None):
    """grad_magnitudes at query rows `rows` (dQ) and keys `keys` (dK, dV),
    from rows and columns of P as in the oracle's sampled backward (key
    mask and block mask (M, bq, bk) as there)."""
    from oracle import attention
    from oracle import backward as ob
    from workloads import to_f64
    q, k, v, do = (to_f64(t) for t in (q, k, v, do))
    rows, keys = np.asarray(rows), np.asarray(keys)
    B, H, N, d = q.shape
    mq = np.zeros((B, H, len(rows), d))
    mk, mv = (np.zeros((B, H, len(keys), d)) for _ in range(2))
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, h], k[b, h], v[b, h], do[b, h]
            kvb = None if key_valid is None else np.asarray(key_valid, dtype=bool)[b]
            o, lse = attention(qh[None, None], kh[None, None], vh[None, None], scale, causal=causal,
                               key_valid=None if kvb is None else kvb[None], block_mask=block_mask)
            delta = np.abs(ob._delta_from_output(doh, o[0, 0]))
            p_r = ob._probabilities(qh, kh, scale, causal, rows, kvb, block_mask)
            mds_r = p_r * (np.abs(ob._dp(doh[rows], vh)) + delta[rows][:, None])
            mq[b, h] = abs(scale) * (mds_r @ np.abs(kh))
            p_c = ob._probability_columns(qh, kh[keys], lse[0, 0], scale, causal, keys,
                                          None if kvb is None else kvb[keys], block_mask)
            mds_c = p_c * (np.abs(ob._dp(doh, vh[keys])) + delta[:, None])
            mk[b, h] = abs(scale) * (mds_c.T @ np.abs(qh))
            mv[b, h] = p_c.T @ np.abs(doh)
    return mq, mk, mv
