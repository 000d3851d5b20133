"""Gradients of exact attention in float64, written as the plain definition.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's CPU
leg, never by the product path.

What is computed (FlashAttention reading notes, section "recomputation"):
the backward pass keeps only O and the softmax statistics of the forward
pass and recomputes the probabilities from Q and K.  Here, for one loss
gradient dO = dL/dO, the gradients follow from O = P V with
P = softmax(S), S = scale * Q K^T (masked):

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij = sum_f dO_if O_if      (row sums)
    dS = P * (dP - D)                               (softmax's Jacobian)
    dQ = scale * dS K
    dK = scale * dS^T Q

A key hidden by a key-padding mask (``key_valid`` False; the forward
oracle's key mask) has probability 0 in every row, so it receives dK = dV = 0
and adds nothing to dQ; a (query, key) pair hidden by a block mask
(``block_mask``, as in the forward oracle) has probability 0 and passes no
gradient between them.  A row that sees no key at all has the constant
output O = 0 (the forward oracle's empty row): its probabilities are all 0,
so it passes no gradient anywhere and its dQ is 0.

The probabilities are recomputed in float64 from the inputs (two passes
over a row, as in ``oracle.fp64``).  Each step is a module-level function
so that the tests can break one at a time.
"""

import numpy as np

from . import fp64


def _probabilities(q, k, scale, causal, rows, key_valid=None, block_mask=None):
    """P [R, N] for query rows `rows` of one head (masked keys give 0; a row
    that sees no key is all 0).  key_valid: bool [N] or None; block_mask:
    (M, bq, bk) or None, as in the forward oracle."""
    s = fp64._scores(q[rows], k, scale)
    vis = fp64._visible(rows, k.shape[0], causal, key_valid)
    if block_mask is not None:
        vis &= fp64._block_visible(rows, k.shape[0], block_mask)
    s = np.where(vis, s, -np.inf)
    empty = fp64._empty_rows(vis)
    m = np.where(empty, 0.0, fp64._row_max(s))
    e = fp64._exp_shifted(s, m)
    l = fp64._row_sum(e)
    return e / np.where(empty, 1.0, l)[:, None]


def _dv(p, do):
    """dV = P^T dO."""
    return p.T @ do


def _dp(do, v):
    """dP = dO V^T."""
    return do @ v.T


def _delta(p, dp):
    """D_i = sum_j P_ij dP_ij."""
    return (p * dp).sum(axis=1)


def _ds(p, dp, delta):
    """dS = P * (dP - D)."""
    return p * (dp - delta[:, None])


def _dq(ds, k, scale):
    """dQ = scale * dS K."""
    return scale * (ds @ k)


def _dk(ds, q, scale):
    """dK = scale * dS^T Q."""
    return scale * (ds.T @ q)


def attention_backward(q, k, v, do, scale, causal=False, key_valid=None, block_mask=None):
    """dQ, dK, dV (float64, [B, H, N, d]) of exact attention for upstream
    gradient dO.  Inputs of any real dtype are converted exactly to f64.
    key_valid: optional bool [B, N], False hides that key from every query;
    block_mask: optional (M, bq, bk), key j hidden from query i when
    M[i // bq][j // bk] == 0 (both as in the forward oracle)."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H, N, d = q.shape
    kv = None if key_valid is None else np.asarray(key_valid, dtype=bool)
    dq, dk, dv = (np.zeros((B, H, N, d)) for _ in range(3))
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            p = _probabilities(q[b, h], k[b, h], scale, causal, rows, None if kv is None else kv[b], block_mask)
            dp = _dp(do[b, h], v[b, h])
            delta = _delta(p, dp)
            ds = _ds(p, dp, delta)
            dv[b, h] = _dv(p, do[b, h])
            dq[b, h] = _dq(ds, k[b, h], scale)
            dk[b, h] = _dk(ds, q[b, h], scale)
    return dq, dk, dv


def _delta_from_output(do, o):
    """D_i = sum_f dO_if O_if (equal to sum_j P_ij dP_ij since O = P V)."""
    return (do * o).sum(axis=1)


def _probability_columns(q, k_cols, lse, scale, causal, cols, cols_valid=None, block_mask=None):
    """P [N, C] at key columns `cols` of one head: exp(S_ij - LSE_i) over
    every query i, with LSE_i the row's log-sum-exp of scaled, masked
    scores (so the column needs no other key).  cols_valid: bool [C] or
    None, False for a column hidden by the key mask (all 0); block_mask:
    (M, bq, bk) or None, a pair whose block of M is 0 gives 0; a query that
    sees the column has a finite LSE."""
    s = fp64._scores(q, k_cols, scale)
    vis = np.ones(s.shape, dtype=bool)
    if causal:
        vis &= cols[None, :] <= np.arange(q.shape[0])[:, None]
    if cols_valid is not None:
        vis &= np.asarray(cols_valid, dtype=bool)[None, :]
    if block_mask is not None:
        vis &= fp64._block_visible(np.arange(q.shape[0]), k_cols.shape[0], block_mask, keys=cols)
    with np.errstate(over="ignore", invalid="ignore"):
        return np.where(vis, np.exp(np.where(vis, s, 0.0) - np.where(vis, lse[:, None], 0.0)), 0.0)


def attention_backward_sampled(q, k, v, do, scale, causal, rows, keys, key_valid=None, block_mask=None):
    """dQ at query rows `rows` and dK, dV at key rows `keys` (float64,
    [B, H, len(rows), d] and [B, H, len(keys), d]): the gradients of
    ``attention_backward`` for a sample of their rows, at sizes where the
    full N x N matrices per head are too large.  Row i of dQ needs row i of
    P and dP (and D_i); row j of dK and dV needs column j of P and dP, and D
    for every query.  O and LSE of every query come from the forward oracle,
    so column j of P is exp(S_ij - LSE_i) and D_i = sum_f dO_if O_if.
    key_valid: optional bool [B, N] key mask and block_mask: optional (M,
    bq, bk) block mask, as in ``attention_backward``."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    kv = None if key_valid is None else np.asarray(key_valid, dtype=bool)
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    B, H, N, d = q.shape
    dq = np.zeros((B, H, len(rows), d))
    dk, dv = (np.zeros((B, H, len(keys), d)) for _ in range(2))
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, h], k[b, h], v[b, h], do[b, h]
            kvb = None if kv is None else kv[b]
            o, lse = fp64.attention(qh[None, None], kh[None, None], vh[None, None], scale, causal=causal,
                                    key_valid=None if kvb is None else kvb[None], block_mask=block_mask)
            delta = _delta_from_output(doh, o[0, 0])
            p_r = _probabilities(qh, kh, scale, causal, rows, kvb, block_mask)
            ds_r = _ds(p_r, _dp(doh[rows], vh), delta[rows])
            dq[b, h] = _dq(ds_r, kh, scale)
            p_c = _probability_columns(qh, kh[keys], lse[0, 0], scale, causal, keys,
                                       None if kvb is None else kvb[keys], block_mask)
            ds_c = _ds(p_c, _dp(doh, vh[keys]), delta)
            dv[b, h] = _dv(p_c, doh)
            dk[b, h] = _dk(ds_c, qh, scale)
    return dq, dk, dv
