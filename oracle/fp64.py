"""Exact attention in float64, written as the plain definition.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.

What is computed (FlashAttention reading notes, section "problem setting"):
for every batch entry b and head h, with Q, K, V each holding N rows of d
features, the output is O = softmax(S) V where S = scale * Q K^T.  The
caller's ``scale`` multiplies the raw dot products before the softmax (the
problem statement on that page carries no scale; the workloads use
1/sqrt(d), which is also what the worked mask example on the Qiita page,
section 6, needs to print the value it prints).

Causal masking: key j is visible to query i iff j <= i.  The pages name a
causal (GPT-2) workload but do not write the convention out; this is the
plainest lower-triangular reading with the diagonal kept, so no row is empty.

Optional ``key_valid`` [B, N] (True = the key takes part) is the additive
-inf key-padding bias described on the Qiita page, section 4 and section 6:
a padded key gets -inf added to its score.  A row that sees no key at all
has no softmax; the pages say nothing about it.  Reading taken here: its row
sum is the empty sum 0, so LSE = ln 0 = -inf, and O is the empty weighted
sum, the zero vector.  These are the values under which merging the results
of two disjoint key sets (the combination rule of the FlashAttention reading
notes, section "proposed method": m = max(m1, m2), l = e^(m1-m) l1 +
e^(m2-m) l2) leaves the other set's result unchanged when one set is empty.

Optional ``block_mask`` (M, bq, bk): the block-sparse variant of the
FlashAttention reading notes, section "block-sparse FlashAttention": a
predefined 0/1 matrix M over (query block, key block) pairs, query blocks of
bq rows and key blocks of bk keys; only the blocks where M is 1 take part,
i.e. key j is hidden from query i when M[i // bq][j // bk] = 0.  The same M
serves every batch entry and head.  It combines with the other masks.

LSE: the forward pass keeps, besides O, the softmax statistics m (row max)
and l (row sum of exp(s - m)) for the backward pass (FlashAttention reading
notes, section "recomputation").  They are returned folded into one number
per row, LSE_i = m_i + ln(l_i), natural log of the scaled, masked scores.

Non-finite inputs are not scrubbed (the pages say nothing about them; the
plainest reading is the definition applied as written): a NaN in a visible
key's K row makes that row's scores, hence its O and LSE, NaN; a NaN in a
visible key's V row makes that feature of O NaN.  A hidden key takes no part
at all: its score is replaced by -inf before the softmax and its V row is
left out of the weighted sum.

Arithmetic: inputs are converted exactly to float64 (bf16 and fp32 values
are exact there); scores, exponentials, sums and the final division are
float64.  The softmax is evaluated in two passes over a full row (max, then
exp and sum) with no online rescaling, so it shares no algorithm with the
tiled GPU kernel beyond the definition itself.

Each step is a small module-level function so that the tests can replace one
step with a plausible mistake and check that the pins catch it.
"""

import math

import numpy as np


def _scores(q, k, scale):
    """S = scale * Q K^T for one head: q [R, d], k [N, d] -> [R, N]."""
    return scale * (q @ k.T)


def _visible(rows, n_keys, causal, key_valid):
    """bool [R, N]: True where key j enters query row rows[r]'s softmax."""
    vis = np.ones((len(rows), n_keys), dtype=bool)
    if causal:
        vis &= np.arange(n_keys)[None, :] <= rows[:, None]
    if key_valid is not None:
        vis &= key_valid[None, :]
    return vis


def _block_visible(rows, n_keys, block_mask, keys=None):
    """bool [R, N]: M[i // bq][j // bk] for query rows[r] and key j (or,
    given ``keys``, bool [R, len(keys)] for those keys only)."""
    m, bq, bk = block_mask
    cols = np.arange(n_keys) if keys is None else np.asarray(keys)
    return np.asarray(m, dtype=bool)[rows[:, None] // bq, cols[None, :] // bk]


def _row_max(s):
    """m_i = max_j s_ij (the softmax's shift; -inf for an empty row)."""
    return s.max(axis=1)


def _exp_shifted(s, m):
    """exp(s_ij - m_i); a masked score (-inf) gives exactly 0."""
    return np.exp(s - m[:, None])


def _row_sum(e):
    """l_i = sum_j exp(s_ij - m_i)."""
    return e.sum(axis=1)


def _weighted_values(e, v, vis):
    """sum_j exp(s_ij - m_i) * v_j over the keys row i sees, before
    normalisation: [R, N] x [N, d].

    A hidden key takes no part in the sum (its -inf bias removes it), so a
    non-finite value in a hidden key's V row never reaches the row.  Keys
    whose V rows are finite go through one matrix product (a hidden key's
    e_ij is exactly 0 there); the few others are summed over the visible
    entries only."""
    fin = np.isfinite(v).all(axis=1)
    out = e[:, fin] @ v[fin]
    if not fin.all():
        eb, vb, visb = e[:, ~fin], v[~fin], vis[:, ~fin]
        out = out + np.where(visb[:, :, None], eb[:, :, None] * vb[None, :, :], 0.0).sum(axis=1)
    return out


def _normalise(o_unnormalised, l):
    """O_i = (sum_j e_ij v_j) / l_i."""
    return o_unnormalised / l[:, None]


def _lse(m, l):
    """LSE_i = m_i + ln l_i (natural log)."""
    return m + np.log(l)


def _empty_rows(vis):
    """Rows that see no key at all."""
    return ~vis.any(axis=1)


def _empty_row_result(o, lse, empty):
    """An empty row: O = 0 (empty weighted sum), LSE = ln 0 = -inf."""
    o = np.where(empty[:, None], 0.0, o)
    lse = np.where(empty, -np.inf, lse)
    return o, lse


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, scale, causal=False, key_valid=None, rows=None,
              row_chunk=512, block_mask=None):
    """Exact attention forward, float64.

    q, k, v: arrays [B, H, N, d] (any real dtype; converted exactly to f64).
    scale:   multiplies Q K^T.
    causal:  hide key j from query i when j > i.
    key_valid: optional bool [B, N]; False hides that key from every query.
    rows:    optional 1-D array of query indices, evaluated for every (b, h);
             default all N rows.  Lets large workloads be checked on a sample.
    block_mask: optional (M, bq, bk): M a 0/1 array [ceil(N/bq), ceil(N/bk)];
             key j is hidden from query i when M[i // bq][j // bk] == 0.
    Returns (o [B, H, R, d], lse [B, H, R]) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    if k.shape != (B, H, N, d) or v.shape != (B, H, N, d):
        raise ValueError("q, k, v must share the shape [B, H, N, d]")
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    kv = None if key_valid is None else np.asarray(key_valid, dtype=bool)
    o = np.empty((B, H, len(rows), d), dtype=np.float64)
    lse = np.empty((B, H, len(rows)), dtype=np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        for b in range(B):
            for h in range(H):
                for c0 in range(0, len(rows), row_chunk):
                    r = rows[c0:c0 + row_chunk]
                    s = _scores(q[b, h, r], k[b, h], scale)
                    vis = _visible(r, N, causal, None if kv is None else kv[b])
                    if block_mask is not None:
                        vis &= _block_visible(r, N, block_mask)
                    s = np.where(vis, s, -np.inf)
                    empty = _empty_rows(vis)
                    m = _row_max(s)
                    m = np.where(empty, 0.0, m)   # any finite shift: every e_ij is 0
                    e = _exp_shifted(s, m)
                    l = _row_sum(e)
                    o_r = _normalise(_weighted_values(e, v[b, h], vis), l)
                    lse_r = _lse(m, l)
                    o_r, lse_r = _empty_row_result(o_r, lse_r, empty)
                    o[b, h, c0:c0 + len(r)] = o_r
                    lse[b, h, c0:c0 + len(r)] = lse_r
    return o, lse


def attention_materialised(q, k, v, scale, causal=False, key_valid=None, block_mask=None):
    """Standard attention with the full score and probability tables.

    This is the "standard attention" the FlashAttention reading notes contrast
    with the method (section "problem setting": S = Q K^T and P = softmax(S)
    both written out in full).  Used only on tiny inputs to cross-check
    ``attention``.  Returns (o, lse, p) with p the [B, H, N, N] probabilities.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    s = scale * np.matmul(q, np.swapaxes(k, -1, -2))          # [B, H, N, N]
    hide = np.zeros((B, 1, N, N), dtype=bool)
    if causal:
        hide |= np.triu(np.ones((N, N), dtype=bool), k=1)[None, None]
    if key_valid is not None:
        hide |= ~np.asarray(key_valid, dtype=bool)[:, None, None, :]
    if block_mask is not None:
        m, bq, bk = block_mask
        m = np.asarray(m, dtype=bool)
        full = np.repeat(np.repeat(m, bq, axis=0), bk, axis=1)[:N, :N]
        hide = hide | ~full[None, None]
    s = np.where(hide, -np.inf, s)
    with np.errstate(invalid="ignore", divide="ignore"):
        top = s.max(axis=-1, keepdims=True)
        w = np.exp(s - top)
        z = w.sum(axis=-1, keepdims=True)
        p = w / z
        o = np.matmul(p, v)
        lse = (top + np.log(z))[..., 0]
    # a row with every key hidden: P row 0, O = 0, LSE = -inf
    empty = np.broadcast_to(hide.all(axis=-1), lse.shape)
    p = np.where(empty[..., None], 0.0, p)
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, lse)
    return o, lse, p


def attention_fsum(q, k, v, scale, causal=False, key_valid=None):
    """Pure-Python attention with every sum exactly rounded (math.fsum).

    Products of two fp32 values are exact in float64, so each dot product is
    the correctly rounded exact value; every later sum is correctly rounded
    too.  The result therefore does not depend on the order of the keys,
    which makes bit-exact permutation checks possible.  Tiny inputs only.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(N)
                        if (not causal or j <= i)
                        and (key_valid is None or key_valid[b][j])]
                if not keys:
                    o[b, h, i] = 0.0
                    lse[b, h, i] = -math.inf
                    continue
                s = {j: scale * math.fsum(q[b, h, i, t] * k[b, h, j, t] for t in range(d))
                     for j in keys}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                z = math.fsum(e.values())
                for t in range(d):
                    o[b, h, i, t] = math.fsum(e[j] * v[b, h, j, t] for j in keys) / z
                lse[b, h, i] = m + math.log(z)
    return o, lse
