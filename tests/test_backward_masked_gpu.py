"""Backward pass with key-padding masks on the GPU (attn_bwd_masked) against
the fp64 oracle's gradients.

A batch entry's keys at or past its valid length are hidden from every
query (the forward's key_len), so by the recomputation of the FlashAttention
reading notes (section "recomputation") their probabilities are 0 in every
row: they get dK = dV = 0 exactly and add nothing to dQ, and an entry with
no valid key (constant output 0) gets all-zero gradients.  O and LSE come
from the GPU's own masked forward, as in a training step.  The bar is the
unmasked backward's (tests/parity.py, GRAD), and the exact zeros must be
exact.
"""

import numpy as np
import pytest
import torch

import exact_attention_29_amd as ea
from oracle import attention_backward, attention_backward_sampled
from tests.parity import assert_grad_within, grad_magnitudes, grad_magnitudes_sampled
from workloads import WORKLOADS, Workload, block_rows, make_inputs, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def inputs(B, H, N, seed, sigma=1.0):
    w = Workload("bwd_mask", B, H, N, 64, "bf16", sigma, 0.125, False, seed, "")
    q, k, v = make_inputs(w)
    do = make_inputs(Workload("bwd_mask_do", B, H, N, 64, "bf16", 1.0, 0.125, False, seed + 1, ""))[0]
    return q, k, v, do


def grads_gpu(q, k, v, do, scale, causal, lengths, valid=None):
    """Forward and backward with valid lengths, or (valid: bool [B, N]) a key
    bit mask, and lengths too unless lengths is None."""
    q, k, v, do = (t.to(DEV) for t in (q, k, v, do))
    masks = {}
    if lengths is not None:
        masks["key_len"] = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    if valid is not None:
        masks["key_valid"] = torch.tensor(valid, device=DEV)
    o, lse = ea.forward(q, k, v, scale=scale, causal=causal, **masks)
    dq, dk, dv = ea.backward(q, k, v, o, lse, do, scale=scale, causal=causal, **masks)
    torch.cuda.synchronize()
    return dq, dk, dv


def key_valid(lengths, n):
    return np.arange(n)[None, :] < np.clip(np.asarray(lengths), 0, n)[:, None]


def check_exact_zeros(dq, dk, dv, valid, what):
    """Hidden keys' dK and dV, and every gradient of an entry with no valid
    key, are exactly 0 (valid: bool [B, N])."""
    kv = torch.tensor(valid, device=dk.device)
    hidden = ~kv[:, None, :, None]
    assert not (dk.float() * hidden).any() and not (dv.float() * hidden).any(), f"{what}: hidden keys' dK/dV"
    for b in range(valid.shape[0]):
        if not valid[b].any():
            assert not dq[b].float().any() and not dk[b].float().any() and not dv[b].float().any(), \
                f"{what}: entry {b} has no valid key"


def compare_full(q, k, v, do, causal, lengths, what, valid=None):
    n = q.shape[2]
    print(f"[case] {what}", flush=True)
    dq, dk, dv = grads_gpu(q, k, v, do, 0.125, causal, lengths, valid)
    kv = np.ones((q.shape[0], n), dtype=bool) if lengths is None else key_valid(lengths, n)
    if valid is not None:
        kv = kv & valid
    ref = attention_backward(to_f64(q), to_f64(k), to_f64(v), to_f64(do), 0.125, causal=causal, key_valid=kv)
    mags = grad_magnitudes(q, k, v, do, 0.125, causal, key_valid=kv)
    for name, g, r, m in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref, mags):
        assert_grad_within(f"{name} {what}", g, r, m)
    check_exact_zeros(dq, dk, dv, kv, what)


@pytest.mark.parametrize("n", [1, 17, 65, 200, 513])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_len_sizes(n, causal):
    """Four entries: every key valid, a single key, a ragged middle length,
    none."""
    q, k, v, do = inputs(4, 2, n, seed=5100 + n)
    compare_full(q, k, v, do, causal, [n, 1, n // 2 + 3, 0], f"n={n} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_len_pipeline_lengths(causal):
    """N = 2,100 (several turns of both kernels' tile rings) cut at lengths
    inside the pipelined stretch, on a tile edge and in the last tile."""
    q, k, v, do = inputs(4, 1, 2100, seed=5200)
    compare_full(q, k, v, do, causal, [700, 1337, 2048, 2099], f"n=2100 causal={causal}")


def _bits(B, n, seed, density=0.7):
    """A random key mask [B, n]: entry 0 at the given density (key 0 kept),
    entry 1 with no valid key, entry 2 with every key valid."""
    rng = np.random.default_rng(seed)
    valid = rng.random((B, n)) < density
    valid[0, 0] = True
    valid[1] = False
    valid[2] = True
    return valid


@pytest.mark.parametrize("n", [1, 33, 65, 300, 1337])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_bits(n, causal):
    """A key bit mask (the forward's key_valid, packed): a random pattern,
    an entry with no valid key, an entry with all keys valid (n = 300 and
    1,337 run pipelined dQ steps, which drop hidden keys through a lane
    mask per register: keys 4 apart in one word go to the two lane
    halves)."""
    q, k, v, do = inputs(3, 2, n, seed=5600 + n)
    compare_full(q, k, v, do, causal, None, f"bits n={n} causal={causal}", valid=_bits(3, n, 5650 + n))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_bits_and_lengths(causal):
    """Both masks at once: a key is hidden when past the length or when its
    bit is clear."""
    q, k, v, do = inputs(3, 2, 700, seed=5700)
    compare_full(q, k, v, do, causal, [500, 700, 333], f"bits and lengths causal={causal}",
                 valid=_bits(3, 700, 5750, density=0.5))


def test_backward_full_lengths_match_unmasked_bitwise():
    """key_len = N everywhere: the same bits as the unmasked backward."""
    q, k, v, do = (t.to(DEV) for t in inputs(2, 3, 777, seed=5300))
    for causal in (False, True):
        o, lse = ea.forward(q, k, v, scale=0.125, causal=causal)
        plain = ea.backward(q, k, v, o, lse, do, scale=0.125, causal=causal)
        kl = torch.full((2,), 777, dtype=torch.int32, device=DEV)
        masked = ea.backward(q, k, v, o, lse, do, scale=0.125, causal=causal, key_len=kl)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(plain, masked)), f"causal={causal}"


def test_backward_key_len_is_clamped():
    """Lengths below 0 or above N act as 0 and N."""
    q, k, v, do = (t.to(DEV) for t in inputs(2, 2, 300, seed=5400))
    clamped = grads_gpu(q, k, v, do, 0.125, False, [0, 300])
    raw = grads_gpu(q, k, v, do, 0.125, False, [-7, 1000])
    assert all(torch.equal(a, b) for a, b in zip(clamped, raw))


def test_backward_key_len_deterministic():
    q, k, v, do = inputs(3, 2, 640, seed=5500)
    a = grads_gpu(q, k, v, do, 0.125, True, [640, 333, 17])
    b = grads_gpu(q, k, v, do, 0.125, True, [640, 333, 17])
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_len_patch_3mp_sampled(causal):
    """The 3 MP patch shape (N = 11,616) with two entries of one head, one
    with 8,000 valid keys: dQ at three random 128-row blocks plus the last,
    dK and dV at three random 128-key blocks plus the last and the block
    holding the last valid key, against the oracle's gradients there."""
    w = WORKLOADS["patch_3mp"]
    q1, k1, v1 = (t[:, :1] for t in make_inputs(w))
    q, k, v = (torch.cat([t, t.flip(2)], 0).contiguous() for t in (q1, k1, v1))
    do = make_inputs(Workload("do", 2, 1, w.N, 64, "bf16", 1.0, w.scale, causal, w.seed + 60, ""))[0]
    lengths = [w.N, 8000]
    print(f"[case] 3 MP key_len={lengths} causal={causal}", flush=True)
    dq, dk, dv = grads_gpu(q, k, v, do, w.scale, causal, lengths)
    rows = block_rows(w.N, 3, seed=83, rows_per_block=128)
    keys = np.unique(np.concatenate([block_rows(w.N, 3, seed=84, rows_per_block=128),
                                     np.arange(7936, 8064)]))
    kv = key_valid(lengths, w.N)
    ref = attention_backward_sampled(to_f64(q), to_f64(k), to_f64(v), to_f64(do), w.scale, causal, rows, keys,
                                     key_valid=kv)
    mags = grad_magnitudes_sampled(q, k, v, do, w.scale, causal, rows, keys, key_valid=kv)
    got = (dq[:, :, rows], dk[:, :, keys], dv[:, :, keys])
    for name, g, r, m in zip(("dQ", "dK", "dV"), got, ref, mags):
        assert_grad_within(f"{name} 3 MP key_len causal={causal}", g, r, m)
    check_exact_zeros(dq, dk, dv, kv, "3 MP")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_bits_patch_3mp_sampled(causal):
    """The 3 MP patch shape (N = 11,616) with two entries of one head under
    key bit masks: entry 0 with a random tenth of its keys hidden, entry 1
    with every fourth 32-key word hidden whole and a random half of another
    word's keys, plus a valid length of 9,000 on entry 1; dQ at three
    random 128-row blocks plus the last, dK and dV at three random 128-key
    blocks plus the last and the block around the length, against the
    oracle's gradients there; hidden keys' dK and dV exactly 0."""
    w = WORKLOADS["patch_3mp"]
    q1, k1, v1 = (t[:, :1] for t in make_inputs(w))
    q, k, v = (torch.cat([t, t.flip(2)], 0).contiguous() for t in (q1, k1, v1))
    do = make_inputs(Workload("do", 2, 1, w.N, 64, "bf16", 1.0, w.scale, causal, w.seed + 62, ""))[0]
    rng = np.random.default_rng(5800)
    valid = np.ones((2, w.N), dtype=bool)
    valid[0] = rng.random(w.N) >= 0.1
    words = np.arange(w.N) // 32
    valid[1] = (words % 4) != 3
    half = (words % 4) == 1
    valid[1, half] = rng.random(int(half.sum())) < 0.5
    lengths = [w.N, 9000]
    print(f"[case] 3 MP key bits + key_len={lengths} causal={causal}", flush=True)
    dq, dk, dv = grads_gpu(q, k, v, do, w.scale, causal, lengths, valid)
    rows = block_rows(w.N, 3, seed=87, rows_per_block=128)
    keys = np.unique(np.concatenate([block_rows(w.N, 3, seed=88, rows_per_block=128), np.arange(8960, 9088)]))
    kv = key_valid(lengths, w.N) & valid
    ref = attention_backward_sampled(to_f64(q), to_f64(k), to_f64(v), to_f64(do), w.scale, causal, rows, keys,
                                     key_valid=kv)
    mags = grad_magnitudes_sampled(q, k, v, do, w.scale, causal, rows, keys, key_valid=kv)
    got = (dq[:, :, rows], dk[:, :, keys], dv[:, :, keys])
    for name, g, r, m in zip(("dQ", "dK", "dV"), got, ref, mags):
        assert_grad_within(f"{name} 3 MP key bits causal={causal}", g, r, m)
    check_exact_zeros(dq, dk, dv, kv, "3 MP bits")
