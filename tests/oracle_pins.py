"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a fact it did not compute itself: a value printed on a page, a closed form,
an invariant of the definition, or another library's routine.  The tests run
every pin against the oracle as it stands, and run the "independent" pins
again against deliberately broken copies of single oracle steps to show that
each plausible mistake is caught.
"""

import json
import math
import os

import numpy as np
import torch

from oracle import fp64 as O
from workloads import WORKLOADS, make_inputs, to_f64

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, atol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= atol, f"{what}: max abs error {err:.3e} > {atol:.1e}"


# ---------------------------------------------------------------- closed forms

def pin_uniform_closed_form():
    """Q = 0 makes every score 0: each row averages the values it can see.

    Non-causal: O_i = mean_j V_j and LSE_i = ln N.  Causal: O_i is the mean of
    V_0..V_i and LSE_i = ln(i + 1).  A small row chunk makes the causal mask
    cross chunk boundaries, so it must use global query indices.
    """
    rng = _rng(1)
    B, H, N, d = 2, 3, 37, 16
    q = np.zeros((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    o, lse = O.attention(q, k, v, 0.3)
    _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), 1e-12, "uniform O")
    _close(lse, np.full((B, H, N), math.log(N)), 1e-12, "uniform LSE")
    o, lse = O.attention(q, k, v, 0.3, causal=True, row_chunk=7)
    counts = np.arange(1, N + 1, dtype=np.float64)
    _close(o, np.cumsum(v, axis=2) / counts[:, None], 1e-12, "causal prefix-mean O")
    _close(lse, np.broadcast_to(np.log(counts), (B, H, N)), 1e-12, "causal LSE = ln(i+1)")


def _identity_probs(beta, n, causal):
    e = math.exp(beta)
    p = np.zeros((n, n))
    for i in range(n):
        seen = i + 1 if causal else n
        z = e + seen - 1
        for j in range(seen):
            p[i, j] = (e if j == i else 1.0) / z
    lse = np.array([math.log(e + (i + 1 if causal else n) - 1) for i in range(n)])
    return p, lse


def pin_identity_closed_form():
    """Q = K = alpha * (first N rows of I_d), V = first N rows of I_d.

    Then s_ij = beta * [i == j] with beta = scale * alpha^2, so
    P_ij = (e^beta [i==j] + [i!=j]) / (e^beta + N - 1), O = P padded with zero
    columns, and LSE_i = ln(e^beta + N - 1).  Causal: row i only sees
    j <= i, so the N above becomes i + 1.  beta = 40 makes LSE ~ 40, which
    exposes an LSE that forgets the row max.
    """
    n, d = 6, 8
    for alpha, scale in ((3.0, 0.7), (8.0, 0.625)):
        beta = scale * alpha * alpha
        eye = np.eye(n, d)[None, None]
        for causal in (False, True):
            p, lse_ref = _identity_probs(beta, n, causal)
            o, lse = O.attention(alpha * eye, alpha * eye, eye, scale, causal=causal)
            o_ref = np.zeros((n, d))
            o_ref[:, :n] = p
            _close(o[0, 0], o_ref, 1e-13, f"identity O beta={beta} causal={causal}")
            _close(lse[0, 0], lse_ref, 1e-12, f"identity LSE beta={beta} causal={causal}")


def pin_single_peak_orientation():
    """Only query i* and key j* (i* != j*) are non-zero, both along feature 0.

    Row i* gives key j* the score beta = scale * gamma and every other key 0;
    every other row is uniform.  Scores of K Q^T instead of Q K^T would put
    the peak in row j*; pairing keys with the wrong values moves it too.
    """
    rng = _rng(2)
    n, d, i_s, j_s, gamma, scale = 9, 4, 2, 6, 5.0, 0.5
    beta = scale * gamma
    q = np.zeros((1, 1, n, d))
    k = np.zeros((1, 1, n, d))
    q[0, 0, i_s, 0] = gamma
    k[0, 0, j_s, 0] = 1.0
    v = rng.standard_normal((1, 1, n, d))
    o, lse = O.attention(q, k, v, scale)
    vv = v[0, 0]
    expect = np.broadcast_to(vv.mean(axis=0), (n, d)).copy()
    expect[i_s] = (math.exp(beta) * vv[j_s] + vv.sum(axis=0) - vv[j_s]) / (math.exp(beta) + n - 1)
    lse_ref = np.full(n, math.log(n))
    lse_ref[i_s] = math.log(math.exp(beta) + n - 1)
    _close(o[0, 0], expect, 1e-13, "single-peak O")
    _close(lse[0, 0], lse_ref, 1e-13, "single-peak LSE")


# ------------------------------------------------------------------ invariants

def pin_constant_values():
    """V = c everywhere gives O = c (rows of P sum to one).

    Main oracle: within a few ulp.  fsum variant with c a power of two:
    bit-exact, since scaling by 2^k commutes with correct rounding.
    """
    rng = _rng(3)
    B, H, N, d = 1, 2, 50, 8
    q, k = rng.standard_normal((2, B, H, N, d))
    for c in (0.375, -2.0):
        for causal in (False, True):
            o, _ = O.attention(q, k, np.full((B, H, N, d), c), 0.125, causal=causal)
            _close(o, np.full_like(o, c), 8 * abs(c) * 2.0 ** -52, f"constant V={c}")
    qs, ks = q[:, :1, :12], k[:, :1, :12]
    o, _ = O.attention_fsum(qs, ks, np.full((1, 1, 12, 8), 0.5), 0.125)
    assert np.all(o == 0.5), "fsum oracle: constant V not bit-exact"


def pin_single_key():
    """N = 1: the only probability is exp(0) = 1, so O = V bit-exactly and
    LSE = scale * q.k."""
    rng = _rng(4)
    q, k, v = rng.standard_normal((3, 2, 3, 1, 16))
    o, lse = O.attention(q, k, v, 0.25)
    assert np.array_equal(o, v), "N=1: O != V"
    ref = np.array([[0.25 * math.fsum(q[b, h, 0] * k[b, h, 0]) for h in range(3)] for b in range(2)])
    _close(lse[..., 0], ref, 1e-13, "N=1 LSE")


def pin_causal_row_zero():
    """Causal row 0 sees only key 0: O_0 = V_0 bit-exactly, LSE_0 = scale*q0.k0."""
    rng = _rng(5)
    q, k, v = rng.standard_normal((3, 1, 2, 20, 8))
    o, lse = O.attention(q, k, v, 0.125, causal=True)
    assert np.array_equal(o[..., 0, :], v[..., 0, :]), "causal row 0: O != V_0"
    ref = [0.125 * math.fsum(q[0, h, 0] * k[0, h, 0]) for h in range(2)]
    _close(lse[0, :, 0], ref, 1e-13, "causal row 0 LSE")


def pin_key_value_permutation():
    """Permuting keys and values together leaves O and LSE unchanged;
    permuting queries permutes the output rows (non-causal)."""
    rng = _rng(6)
    B, H, N, d = 1, 2, 40, 8
    q, k, v = rng.standard_normal((3, B, H, N, d))
    perm = rng.permutation(N)
    o, lse = O.attention(q, k, v, 0.4)
    o2, lse2 = O.attention(q, k[:, :, perm], v[:, :, perm], 0.4)
    _close(o2, o, 1e-13, "key/value permutation O")
    _close(lse2, lse, 1e-13, "key/value permutation LSE")
    o3, lse3 = O.attention(q[:, :, perm], k, v, 0.4)
    _close(o3, o[:, :, perm], 1e-13, "query permutation O")
    _close(lse3, lse[:, :, perm], 1e-13, "query permutation LSE")
    qs, ks, vs = q[:, :1, :10], k[:, :1, :10], v[:, :1, :10]
    p = perm[perm < 10]
    a = O.attention_fsum(qs, ks, vs, 0.4)
    b = O.attention_fsum(qs, ks[:, :, p], vs[:, :, p], 0.4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "fsum: permutation not bit-exact"


def pin_score_shift():
    """Adding one vector w to every key adds scale*q_i.w to row i's scores:
    O is unchanged and LSE_i grows by exactly that amount."""
    rng = _rng(7)
    B, H, N, d = 1, 2, 30, 8
    q, k, v = rng.standard_normal((3, B, H, N, d))
    w = 3.0 * rng.standard_normal(d)
    for causal in (False, True):
        o, lse = O.attention(q, k, v, 0.5, causal=causal)
        o2, lse2 = O.attention(q, k + w, v, 0.5, causal=causal)
        _close(o2, o, 1e-12, "score shift O")
        _close(lse2 - lse, 0.5 * (q @ w), 1e-12, "score shift LSE")


def pin_one_hot_limit():
    """A score 900 above the rest: O_i = V_argmax and LSE_i = 900 up to
    e^-850.  Any evaluation that exponentiates unshifted scores overflows."""
    rng = _rng(8)
    n, d = 8, 4
    q = 0.1 * rng.standard_normal((1, 1, n, d))
    k = 0.1 * rng.standard_normal((1, 1, n, d))
    q[0, 0, 0] = [30.0, 0.0, 0.0, 0.0]
    k[0, 0, 3] = [30.0, 0.0, 0.0, 0.0]
    v = rng.standard_normal((1, 1, n, d))
    o, lse = O.attention(q, k, v, 1.0)
    _close(o[0, 0, 0], v[0, 0, 3], 1e-40, "one-hot O")
    _close(lse[0, 0, 0], 900.0 + 0.0, 1e-12, "one-hot LSE")


# ------------------------------------------------------ printed worked example

def pin_page_mask_example():
    """Qiita page, section 6: with q = k = v drawn by torch.manual_seed(0);
    torch.randn(1, 2, 4, 8) and key 3 padded, the inverted boolean mask
    matches the additive -inf reference (0.0) and the un-inverted one, which
    attends only to key 3, differs by 3.46 at most.  Only scale 1/sqrt(8)
    prints 3.46, so this also pins the default-scale reading."""
    with open(os.path.join(GOLDEN, "mask_polarity_example.json")) as f:
        g = json.load(f)
    gen = torch.Generator().manual_seed(0)
    x = torch.randn(1, 2, 4, 8, generator=gen).double().numpy()
    keep = np.array([[True, True, True, False]])
    scale = 1.0 / math.sqrt(8)
    ref, _ = O.attention(x, x, x, scale, key_valid=keep)
    inv, _ = O.attention(x, x, x, scale, key_valid=keep)
    asis, _ = O.attention(x, x, x, scale, key_valid=~keep)
    digits = g["printed_decimals"]
    got_inv = round(float(np.max(np.abs(inv - ref))), digits)
    got_asis = round(float(np.max(np.abs(asis - ref))), digits)
    assert got_inv == g["cases"]["inverted_boolean_mask_attends_keys_0_1_2"], got_inv
    assert got_asis == g["cases"]["boolean_mask_as_is_attends_only_key_3"], got_asis


# ----------------------------------------------------------- library routines

def pin_torch_sdpa_float64():
    """torch's own float64 scaled_dot_product_attention (CPU) and
    torch.logsumexp of the masked scores agree with the oracle."""
    import torch.nn.functional as F
    rng = _rng(9)
    B, H, N, d = 2, 3, 45, 16
    q, k, v = (torch.from_numpy(a) for a in rng.standard_normal((3, B, H, N, d)))
    keep = rng.random((B, N)) > 0.3
    keep[:, 0] = True
    for causal in (False, True):
        for kv in (None, keep):
            o, lse = O.attention(q.numpy(), k.numpy(), v.numpy(), 0.3, causal=causal, key_valid=kv)
            mask = torch.ones(B, 1, N, N, dtype=torch.bool)
            if causal:
                mask &= torch.ones(N, N, dtype=torch.bool).tril()
            if kv is not None:
                mask &= torch.from_numpy(kv)[:, None, None, :]
            ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=0.3)
            s = (0.3 * (q @ k.transpose(-1, -2))).masked_fill(~mask, float("-inf"))
            _close(o, ref.numpy(), 1e-12, f"SDPA f64 causal={causal} mask={kv is not None}")
            _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, "logsumexp f64")


# ------------------------------------------------------- other implementations

def pin_backward_torch_autograd():
    """torch's float64 autograd through the materialised softmax attention
    (a library routine) agrees with the backward oracle."""
    from oracle.backward import attention_backward
    rng = _rng(26)
    B, H, N, d = 2, 2, 33, 16
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    # a key-padding mask per batch entry (key 0 always valid, so no row of
    # torch's SDPA is empty)
    key_valid = rng.random((B, N)) < 0.7
    key_valid[:, 0] = True
    key_valid[1, N // 2:] = False
    for causal in (False, True):
        for kv in (None, key_valid):
            tq, tk, tv = (torch.tensor(t, requires_grad=True) for t in (q, k, v))
            mask = torch.ones(1, 1, N, N, dtype=torch.bool)
            if causal:
                mask = mask & torch.ones(N, N, dtype=torch.bool).tril()
            if kv is not None:
                mask = mask & torch.tensor(kv)[:, None, None, :]
            out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.3)
            out.backward(torch.tensor(do))
            dq, dk, dv = attention_backward(q, k, v, do, 0.3, causal=causal, key_valid=kv)
            what = f"causal={causal}, key mask={kv is not None}"
            _close(dq, tq.grad.numpy(), 1e-11, f"dQ vs torch autograd ({what})")
            _close(dk, tk.grad.numpy(), 1e-11, f"dK vs torch autograd ({what})")
            _close(dv, tv.grad.numpy(), 1e-11, f"dV vs torch autograd ({what})")


def pin_materialised_brute_force():
    """The materialised (standard) attention agrees on the tiny workload and
    on random small shapes; its rows of P sum to one."""
    w = WORKLOADS["tiny"]
    q, k, v = (to_f64(t) for t in make_inputs(w))
    cases = [(q, k, v, w.scale)]
    rng = _rng(10)
    for n, d in ((1, 8), (5, 3), (33, 16), (64, 64), (65, 8)):
        cases.append(tuple(rng.standard_normal((3, 2, 2, n, d))) + (0.2,))
    for q, k, v, scale in cases:
        for causal in (False, True):
            o, lse = O.attention(q, k, v, scale, causal=causal, row_chunk=17)
            ob, lb, p = O.attention_materialised(q, k, v, scale, causal=causal)
            _close(o, ob, 1e-12, f"brute force O n={q.shape[2]} causal={causal}")
            _close(lse, lb, 1e-12, f"brute force LSE n={q.shape[2]} causal={causal}")
            _close(p.sum(axis=-1), np.ones(p.shape[:-1]), 1e-14 * q.shape[2], "rows of P")
    # block masks: the materialised table with blocks cut out
    q, k, v = (rng.standard_normal((2, 2, 37, 8)) for _ in range(3))
    m = rng.random((5, 10)) < 0.6
    m[:, 0] = True  # every row keeps a key
    for causal in (False, True):
        o, lse = O.attention(q, k, v, 0.3, causal=causal, block_mask=(m, 8, 4), row_chunk=9)
        ob, lb, _ = O.attention_materialised(q, k, v, 0.3, causal=causal, block_mask=(m, 8, 4))
        _close(o, ob, 1e-12, f"brute force block-sparse O causal={causal}")
        _close(lse, lb, 1e-12, f"brute force block-sparse LSE causal={causal}")


def pin_fsum_variant():
    """The exactly rounded pure-Python variant agrees on tiny shapes."""
    rng = _rng(11)
    for n, d, causal in ((1, 4, False), (7, 5, True), (16, 8, False), (13, 6, True)):
        q, k, v = rng.standard_normal((3, 1, 2, n, d))
        o, lse = O.attention(q, k, v, 0.35, causal=causal)
        of, lf = O.attention_fsum(q, k, v, 0.35, causal=causal)
        _close(o, of, 1e-14, "fsum O")
        _close(lse, lf, 1e-14, "fsum LSE")


def pin_row_sampling():
    """Evaluating a subset of rows gives those rows of the full result."""
    rng = _rng(12)
    q, k, v = rng.standard_normal((3, 1, 2, 70, 8))
    rows = np.array([0, 5, 63, 64, 69])
    for causal in (False, True):
        o, lse = O.attention(q, k, v, 0.3, causal=causal)
        os_, ls = O.attention(q, k, v, 0.3, causal=causal, rows=rows, row_chunk=2)
        _close(os_, o[:, :, rows], 1e-14, "sampled rows O")
        _close(ls, lse[:, :, rows], 1e-14, "sampled rows LSE")


def pin_backward_row_sampling():
    """The sampled gradients (dQ at some query rows, dK and dV at some keys,
    from the forward oracle's O and LSE) are those rows of the full backward
    oracle, for ragged, causal and single-key shapes, under key-padding
    masks (hidden sampled keys, an entry with no valid key) and under block
    masks (a query block and a key block with no set block)."""
    from oracle.backward import attention_backward, attention_backward_sampled
    rng = _rng(13)
    for n, causal, masked in ((70, False, False), (70, True, False), (37, True, False), (1, False, False),
                              (70, False, True), (37, True, True)):
        q, k, v, do = rng.standard_normal((4, 2, 2, n, 8))
        rows = np.array(sorted({0, n // 3, n - 1}))
        keys = np.array(sorted({0, n // 2, n - 1}))
        kv = None
        if masked:
            kv = np.ones((2, n), dtype=bool)
            kv[0, n // 2:] = False
            kv[1, :] = False
        dq, dk, dv = attention_backward(q, k, v, do, 0.4, causal=causal, key_valid=kv)
        sq, sk, sv = attention_backward_sampled(q, k, v, do, 0.4, causal, rows, keys, key_valid=kv)
        # absolute: with one key the gradients of Q and K cancel to zero
        for got, ref, what in ((sq, dq[:, :, rows], "dQ"), (sk, dk[:, :, keys], "dK"),
                               (sv, dv[:, :, keys], "dV")):
            assert np.abs(got - ref).max() <= 1e-12, f"sampled {what} (n={n}, causal={causal}, masked={masked})"
    for n, causal in ((70, False), (70, True), (45, True)):
        q, k, v, do = rng.standard_normal((4, 2, 2, n, 8))
        m = rng.random((-(-n // 16), -(-n // 8))) < 0.5
        m[1, :] = False  # queries 16..31 see no key
        m[:, 2] = False  # keys 16..23 are seen by no query
        bm = (m, 16, 8)
        rows = np.array(sorted({0, 20, n // 2, n - 1}))
        keys = np.array(sorted({0, 18, n // 2, n - 1}))
        dq, dk, dv = attention_backward(q, k, v, do, 0.4, causal=causal, block_mask=bm)
        sq, sk, sv = attention_backward_sampled(q, k, v, do, 0.4, causal, rows, keys, block_mask=bm)
        for got, ref, what in ((sq, dq[:, :, rows], "dQ"), (sk, dk[:, :, keys], "dK"),
                               (sv, dv[:, :, keys], "dV")):
            assert np.abs(got - ref).max() <= 1e-12, f"sampled {what} (n={n}, causal={causal}, block mask)"


def _merge(o1, l1, o2, l2):
    """Combine the results of two disjoint key sets (the blockwise rule of the
    FlashAttention reading notes, section "proposed method", written with
    LSE = m + ln l): LSE = ln(e^LSE1 + e^LSE2), O = sum_g e^(LSE_g - LSE) O_g."""
    lse = np.logaddexp(l1, l2)
    w1 = np.exp(l1 - lse)[..., None]
    w2 = np.exp(l2 - lse)[..., None]
    return w1 * o1 + w2 * o2, lse


def pin_key_shard_merge():
    """Hiding complementary key sets and merging the two results gives the
    unmasked result, for random sets and for the split where one set is empty
    (whose result must then be O = 0, LSE = -inf: nothing else leaves the
    merge unchanged).  Causal masking on top must combine the same way."""
    rng = _rng(21)
    B, H, N, d = 2, 2, 23, 8
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    for causal in (False, True):
        full_o, full_l = O.attention(q, k, v, 0.4, causal=causal)
        for split in ("random", "empty"):
            a = rng.random((B, N)) < 0.5 if split == "random" else np.ones((B, N), dtype=bool)
            oa, la = O.attention(q, k, v, 0.4, causal=causal, key_valid=a)
            ob, lb = O.attention(q, k, v, 0.4, causal=causal, key_valid=~a)
            if split == "empty":
                assert np.all(ob == 0.0) and np.all(lb == -np.inf), "empty key set: O = 0, LSE = -inf"
            with np.errstate(invalid="ignore", divide="ignore"):
                o, l = _merge(oa, la, ob, lb)
            # rows empty in both shards cannot occur: the union is every key
            _close(o, full_o, 1e-12, f"merged O ({split}, causal={causal})")
            _close(l, full_l, 1e-12, f"merged LSE ({split}, causal={causal})")


def pin_padding_prefix_uniform():
    """Key padding as a valid prefix of length L_b per batch entry, with Q = 0:
    a row averages V over the first L_b keys and LSE = ln L_b; with L_b = 0 the
    row sees nothing: O = 0, LSE = -inf.  Causal rows see min(i+1, L_b) keys."""
    rng = _rng(22)
    B, H, N, d = 4, 2, 19, 8
    lens = np.array([19, 7, 1, 0])
    valid = np.arange(N)[None, :] < lens[:, None]
    q = np.zeros((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    for causal in (False, True):
        o, lse = O.attention(q, k, v, 0.7, causal=causal, key_valid=valid, row_chunk=5)
        for b in range(B):
            for i in range(N):
                cnt = min(i + 1, lens[b]) if causal else lens[b]
                if cnt == 0:
                    assert np.all(o[b, :, i] == 0.0) and np.all(lse[b, :, i] == -np.inf), \
                        f"padding: empty row b={b} i={i}"
                    continue
                _close(o[b, :, i], v[b, :, :cnt].mean(axis=1), 1e-12, f"padding O b={b} i={i}")
                _close(lse[b, :, i], np.full(H, math.log(cnt)), 1e-12, f"padding LSE b={b} i={i}")


def pin_block_sparse():
    """Block-sparse attention (FlashAttention reading notes, section
    "block-sparse FlashAttention") against facts that do not use it:
    an all-ones M is dense attention; an M that gives each query block one
    key block (a permutation) is dense attention of those rows against those
    keys alone; and complementary masks M, 1-M merge (blockwise rule) into
    the dense result."""
    rng = _rng(23)
    B, H, N, d = 2, 2, 40, 8
    bq, bk = 8, 4
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    nbq, nbk = -(-N // bq), -(-N // bk)
    dense_o, dense_l = O.attention(q, k, v, 0.5)
    o, l = O.attention(q, k, v, 0.5, block_mask=(np.ones((nbq, nbk)), bq, bk))
    _close(o, dense_o, 1e-12, "all-ones M O")
    _close(l, dense_l, 1e-12, "all-ones M LSE")
    # one key block per query block, a permutation c(i) != i: query block i
    # (8 rows) sees exactly the 8 keys of block c(i), given at 8 x 8 and at
    # 8 x 4 granularity (two 4-key blocks); equal to dense attention of those
    # rows against those keys alone.  A small row chunk makes the block rows
    # cross chunk boundaries (global query indices).
    perm = [(3 * i + 1) % nbq for i in range(nbq)]
    m88 = np.zeros((nbq, nbq), dtype=bool)
    m84 = np.zeros((nbq, nbk), dtype=bool)
    for i, c in enumerate(perm):
        m88[i, c] = True
        m84[i, 2 * c] = m84[i, 2 * c + 1] = True
    for m, b_k in ((m88, 8), (m84, 4)):
        o, l = O.attention(q, k, v, 0.5, block_mask=(m, bq, b_k), row_chunk=7)
        for i, c in enumerate(perm):
            rs, ks = slice(i * bq, (i + 1) * bq), slice(c * bq, (c + 1) * bq)
            so, sl_l = O.attention(q[:, :, rs], k[:, :, ks], v[:, :, ks], 0.5)
            _close(o[:, :, rs], so, 1e-12, f"permuted blocks O block {i} (bk={b_k})")
            _close(l[:, :, rs], sl_l, 1e-12, f"permuted blocks LSE block {i} (bk={b_k})")
    # complementary masks merge back to dense, causal or not
    m = rng.random((nbq, nbk)) < 0.5
    for causal in (False, True):
        full_o, full_l = O.attention(q, k, v, 0.5, causal=causal)
        oa, la = O.attention(q, k, v, 0.5, causal=causal, block_mask=(m, bq, bk), row_chunk=11)
        ob, lb = O.attention(q, k, v, 0.5, causal=causal, block_mask=(~m, bq, bk), row_chunk=11)
        with np.errstate(invalid="ignore", divide="ignore"):
            mo, ml = _merge(oa, la, ob, lb)
        _close(mo, full_o, 1e-12, f"merged block-sparse O causal={causal}")
        _close(ml, full_l, 1e-12, f"merged block-sparse LSE causal={causal}")


def pin_backward_finite_differences():
    """The gradients of L = sum(dO * O) against central finite differences of
    the forward oracle (step 1e-6, float64): every entry of dQ, dK and dV,
    causal or not, with and without a key-padding mask (one batch entry with
    two hidden keys, one with every key hidden: its output is the constant
    0, so all its gradients are 0), on a tiny problem."""
    from oracle.backward import attention_backward
    rng = _rng(24)
    B, H, N, d = 2, 2, 6, 4
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    scale, h = 0.7, 1e-6
    key_valid = np.ones((B, N), dtype=bool)
    key_valid[0, [1, 4]] = False
    key_valid[1, :] = False
    for causal, kv in ((False, None), (True, None), (False, key_valid), (True, key_valid)):
        dq, dk, dv = attention_backward(q, k, v, do, scale, causal=causal, key_valid=kv)

        def loss(qq, kk, vv):
            return float((O.attention(qq, kk, vv, scale, causal=causal, key_valid=kv)[0] * do).sum())

        for name, x, g in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [xp if t is x else t for t in (q, k, v)]
                args_m = [xm if t is x else t for t in (q, k, v)]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(g, num, 1e-7, f"{name} vs finite differences (causal={causal}, key mask={kv is not None})")


def pin_backward_invariants():
    """Facts of the softmax: dQ and dK rows do not change when every key's
    score moves by the same amount (adding a constant to a row of S leaves P
    alone), dV's column sums equal dO's (rows of P sum to one), and
    sum_j dS_ij = 0 shows up as dK summing to zero over keys when Q rows are
    equal."""
    from oracle.backward import attention_backward
    rng = _rng(25)
    B, H, N, d = 2, 2, 9, 5
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, 0.6)
    _close(dv.sum(axis=2), do.sum(axis=2), 1e-12, "column sums of dV = column sums of dO")
    # equal query rows: dS rows sum to zero, so the keys' gradients sum to zero
    q_eq = np.broadcast_to(q[:, :, :1], q.shape).copy()
    _, dk_eq, _ = attention_backward(q_eq, k, v, do, 0.6)
    _close(dk_eq.sum(axis=2), np.zeros((B, H, d)), 1e-12, "sum over keys of dK with equal queries")
    # a key shift along q's direction... a shared shift of every key by a
    # vector u moves row i's scores by scale * q_i . u, a per-row constant:
    u = rng.standard_normal(d)
    dq2, dk2, dv2 = attention_backward(q, k + u, v, do, 0.6)
    _close(dv2, dv, 1e-12, "dV under a shared key shift")
    _close(dk2, dk, 1e-12, "dK under a shared key shift")


def pin_backward_block_mask():
    """A block mask in the gradients: against central finite differences of
    the forward oracle with that block mask (every entry, causal or not, a
    mask with a query block that sees no key block), and all-ones M gives the
    unmasked gradients bit for bit."""
    from oracle.backward import attention_backward
    rng = _rng(28)
    B, H, N, d = 1, 2, 8, 4
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    scale, h = 0.6, 1e-6
    m = np.array([[1, 0, 1, 0], [0, 1, 1, 0], [0, 0, 0, 0], [1, 1, 0, 1]], dtype=np.uint8)  # 2-row, 2-key blocks
    for causal in (False, True):
        bm = (m, 2, 2)
        dq, dk, dv = attention_backward(q, k, v, do, scale, causal=causal, block_mask=bm)

        def loss(qq, kk, vv):
            return float((O.attention(qq, kk, vv, scale, causal=causal, block_mask=bm)[0] * do).sum())

        for name, x, g in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [xp if t is x else t for t in (q, k, v)]
                args_m = [xm if t is x else t for t in (q, k, v)]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(g, num, 1e-7, f"{name} vs finite differences (block mask, causal={causal})")
        assert not dq[:, :, 4:6].any(), "a query block that sees no key block has dQ = 0"
        ones = (np.ones_like(m), 2, 2)
        full = attention_backward(q, k, v, do, scale, causal=causal)
        for a, b in zip(attention_backward(q, k, v, do, scale, causal=causal, block_mask=ones), full):
            assert np.array_equal(a, b), f"all-ones block mask (causal={causal})"


def pin_backward_hidden_keys():
    """A key-padding mask in the gradients: the hidden keys' K and V can be
    anything (every gradient stays the same bits), their own dK and dV are
    exactly 0, a batch entry with no valid key gets all-zero gradients, and
    the column sums of dV equal those of dO over the rows that see a key
    (each such row of P sums to one)."""
    from oracle.backward import attention_backward
    rng = _rng(27)
    B, H, N, d = 3, 2, 11, 5
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    key_valid = np.ones((B, N), dtype=bool)
    key_valid[0, 7:] = False            # right padding
    key_valid[1, [0, 3, 4, 9]] = False  # scattered
    key_valid[2, :] = False             # nothing valid
    for causal in (False, True):
        dq, dk, dv = attention_backward(q, k, v, do, 0.45, causal=causal, key_valid=key_valid)
        k2, v2 = k.copy(), v.copy()
        hid = ~key_valid[:, None, :, None] & np.ones((B, H, N, d), dtype=bool)
        k2[hid] = 40.0 * rng.standard_normal(int(hid.sum()))
        v2[hid] = -7.0
        dq2, dk2, dv2 = attention_backward(q, k2, v2, do, 0.45, causal=causal, key_valid=key_valid)
        for name, a, b in (("dQ", dq, dq2), ("dK", dk, dk2), ("dV", dv, dv2)):
            assert np.array_equal(a, b), f"{name} depends on hidden keys (causal={causal})"
        assert not dk[hid].any() and not dv[hid].any(), f"hidden keys get a gradient (causal={causal})"
        assert not dq[2].any() and not dk[2].any() and not dv[2].any(), "entry with no valid key"
        sees = np.array([[(key_valid[b] & ((np.arange(N) <= i) if causal else True)).any() for i in range(N)]
                         for b in range(B)])
        want = (do * sees[:, None, :, None]).sum(axis=2)
        _close(dv.sum(axis=2), want, 1e-12, f"column sums of dV under a key mask (causal={causal})")


def pin_nonfinite_inputs():
    """What a NaN in Q, K or V does under the definition.  Causal rows i < j
    never see key j, so NaN in K_j and V_j leaves them exactly as with finite
    values, while rows i >= j (whose scores include q_i . k_j) are NaN in O
    and LSE.  A key hidden by the padding mask takes no part either.  A NaN
    in feature f of a visible V row makes column f of O NaN and leaves the
    other features and LSE alone (features of O are independent)."""
    rng = _rng(26)
    B, H, N, d, j, f = 1, 2, 11, 8, 6, 3
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    k_bad, v_bad = k.copy(), v.copy()
    k_bad[:, :, j] = np.nan
    v_bad[:, :, j] = np.nan
    with np.errstate(invalid="ignore"):
        ref_o, ref_l = O.attention(q, k, v, 0.4, causal=True, row_chunk=4)
        o, lse = O.attention(q, k_bad, v_bad, 0.4, causal=True, row_chunk=4)
    _close(o[:, :, :j], ref_o[:, :, :j], 1e-12, "causal rows before a NaN key")
    _close(lse[:, :, :j], ref_l[:, :, :j], 1e-12, "causal LSE before a NaN key")
    assert np.isnan(o[:, :, j:]).all() and np.isnan(lse[:, :, j:]).all(), "rows that see a NaN key"
    valid = np.ones((B, N), dtype=bool)
    valid[:, j] = False
    with np.errstate(invalid="ignore"):
        ref_o, ref_l = O.attention(q, k, v, 0.4, key_valid=valid)
        o, lse = O.attention(q, k_bad, v_bad, 0.4, key_valid=valid)
    _close(o, ref_o, 1e-12, "a padded NaN key")
    _close(lse, ref_l, 1e-12, "LSE with a padded NaN key")
    v_one = v.copy()
    v_one[:, :, j, f] = np.nan
    with np.errstate(invalid="ignore"):
        ref_o, ref_l = O.attention(q, k, v, 0.4)
        o, lse = O.attention(q, k, v_one, 0.4)
    assert np.isnan(o[..., f]).all(), "a NaN value reaches its feature in every row"
    keep = [g for g in range(d) if g != f]
    _close(o[..., keep], ref_o[..., keep], 1e-12, "the other features")
    _close(lse, ref_l, 1e-12, "LSE with a NaN value")


INDEPENDENT_PINS = [
    pin_uniform_closed_form,
    pin_identity_closed_form,
    pin_single_peak_orientation,
    pin_constant_values,
    pin_single_key,
    pin_causal_row_zero,
    pin_key_value_permutation,
    pin_score_shift,
    pin_one_hot_limit,
    pin_page_mask_example,
    pin_key_shard_merge,
    pin_padding_prefix_uniform,
    pin_block_sparse,
    pin_backward_finite_differences,
    pin_backward_invariants,
    pin_backward_hidden_keys,
    pin_backward_block_mask,
    pin_nonfinite_inputs,
]

ALL_PINS = INDEPENDENT_PINS + [
    pin_backward_torch_autograd,
    pin_torch_sdpa_float64,
    pin_materialised_brute_force,
    pin_fsum_variant,
    pin_row_sampling,
    pin_backward_row_sampling,
]
