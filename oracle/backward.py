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

The probabilities are recomputed in float64 from the inputs (two passes
over a row, as in ``oracle.fp64``).  Each step is a module-level function
so that the tests can break one at a time.
"""

import numpy as np

from . import fp64


def _probabilities(q, k, scale, causal, rows):
    """P [R, N] for query rows `rows` of one head (masked keys give 0)."""
    s = fp64._scores(q[rows], k, scale)
    vis = fp64._visible(rows, k.shape[0], causal, None)
    s = np.where(vis, s, -np.inf)
    m = fp64._row_max(s)
    e = fp64._exp_shifted(s, m)
    return e / fp64._row_sum(e)[:, None]


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


def attention_backward(q, k, v, do, scale, causal=False):
    """dQ, dK, dV (float64, [B, H, N, d]) of exact attention for upstream
    gradient dO.  Inputs of any real dtype are converted exactly to f64."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H, N, d = q.shape
    dq, dk, dv = (np.zeros((B, H, N, d)) for _ in range(3))
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            p = _probabilities(q[b, h], k[b, h], scale, causal, rows)
            dp = _dp(do[b, h], v[b, h])
            delta = _delta(p, dp)
            ds = _ds(p, dp, delta)
            dv[b, h] = _dv(p, do[b, h])
            dq[b, h] = _dq(ds, k[b, h], scale)
            dk[b, h] = _dk(ds, q[b, h], scale)
    return dq, dk, dv
