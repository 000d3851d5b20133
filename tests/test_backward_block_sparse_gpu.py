"""Block-sparse backward on the GPU (attn_bwd_block_sparse) against the fp64
oracle's gradients.

The forward ran attn_fwd_block_sparse with the same block mask M
([ceil(N/128)][ceil(N/64)], one for every head; query block i / 128, key
block j / 64).  A pair whose block of M is 0 has probability 0 and passes
no gradient between query and key (FlashAttention reading notes, section on
block-sparse FlashAttention: the backward skips the same blocks); a query
whose row of M leaves it no key has O = 0 and gets dQ = 0.  The bar is the
dense backward's (tests/parity.py, GRAD).
"""

import numpy as np
import pytest
import torch

import exact_attention_29_amd as ea
from oracle import attention_backward, attention_backward_sampled
from tests.parity import assert_grad_within, grad_magnitudes_blocks, grad_magnitudes_sampled
from workloads import WORKLOADS, Workload, block_rows, make_inputs, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def inputs(B, H, N, seed):
    w = Workload("bwd_bs", B, H, N, 64, "bf16", 1.0, 0.125, False, seed, "")
    q, k, v = make_inputs(w)
    do = make_inputs(Workload("bwd_bs_do", B, H, N, 64, "bf16", 1.0, 0.125, False, seed + 1, ""))[0]
    return q, k, v, do


def random_mask(n, density, seed, empty_row=True, empty_col=True):
    rng = np.random.default_rng(seed)
    m = (rng.random(((n + 127) // 128, (n + 63) // 64)) < density).astype(np.uint8)
    if empty_row and m.shape[0] > 1:
        m[1] = 0            # a query block that sees no key block
    if empty_col and m.shape[1] > 2:
        m[:, 2] = 0         # a key block no query sees
    return m


def run(q, k, v, do, causal, m):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    md = torch.tensor(m, device=DEV)
    o, lse = ea.forward(qd, kd, vd, scale=0.125, causal=causal, block_mask=md)
    grads = ea.backward(qd, kd, vd, o, lse, dod, scale=0.125, causal=causal, block_mask=md)
    torch.cuda.synchronize()
    return grads


def compare(q, k, v, do, causal, m, what):
    print(f"[case] {what}", flush=True)
    grads = run(q, k, v, do, causal, m)
    bm = (m, 128, 64)
    ref = attention_backward(to_f64(q), to_f64(k), to_f64(v), to_f64(do), 0.125, causal=causal, block_mask=bm)
    mags = grad_magnitudes_blocks(q, k, v, do, 0.125, causal, bm)
    for name, g, r, mg in zip(("dQ", "dK", "dV"), grads, ref, mags):
        assert_grad_within(f"{name} {what}", g, r, mg)
    return grads, ref


@pytest.mark.parametrize("n", [64, 300, 1000, 2100])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_block_sparse_matches_oracle(n, causal):
    """Random masks at half density with an empty query block and an empty
    key block; lengths with a ragged last tile and several turns of the
    rings."""
    q, k, v, do = inputs(1, 2, n, seed=6100 + n)
    m = random_mask(n, 0.5, seed=6150 + n)
    grads, ref = compare(q, k, v, do, causal, m, f"n={n} causal={causal}")
    if m.shape[0] > 1:
        assert not grads[0][:, :, 128:256].float().any(), "a query block with no key block has dQ = 0"


@pytest.mark.parametrize("density", [0.1, 0.9])
def test_backward_block_sparse_densities(density):
    q, k, v, do = inputs(2, 2, 1500, seed=6200)
    compare(q, k, v, do, False, random_mask(1500, density, seed=6210, empty_row=False, empty_col=False),
            f"density={density}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_all_blocks_set_matches_dense(causal):
    """Every block set: the dense gradients, within the bar (the sparse
    kernels run their general path)."""
    q, k, v, do = (t.to(DEV) for t in inputs(1, 3, 777, seed=6300))
    m = torch.ones(((777 + 127) // 128, (777 + 63) // 64), dtype=torch.uint8, device=DEV)
    o, lse = ea.forward(q, k, v, scale=0.125, causal=causal)
    dense = ea.backward(q, k, v, o, lse, do, scale=0.125, causal=causal)
    sparse = ea.backward(q, k, v, o, lse, do, scale=0.125, causal=causal, block_mask=m)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), sparse, dense):
        err = (a.float() - b.float()).abs().max().item()
        ref = b.float().abs().max().item()
        assert err <= 2e-2 * ref, f"{name}: {err} vs max {ref}"


def test_backward_empty_mask_gives_zero():
    """M = 0 everywhere: no query sees a key, every gradient is 0."""
    q, k, v, do = inputs(1, 2, 500, seed=6400)
    m = np.zeros(((500 + 127) // 128, (500 + 63) // 64), dtype=np.uint8)
    for causal in (False, True):
        grads = run(q, k, v, do, causal, m)
        assert all(not g.float().any() for g in grads), f"causal={causal}"


def test_backward_block_sparse_deterministic():
    q, k, v, do = inputs(1, 2, 900, seed=6500)
    m = random_mask(900, 0.4, seed=6510)
    a = run(q, k, v, do, True, m)
    b = run(q, k, v, do, True, m)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_block_sparse_patch_3mp_sampled(causal):
    """The 3 MP patch shape (N = 11,616, one head) under a random block mask
    at half density with an empty query block and an empty key block, the
    launch configuration of the block-sparse bench lines: dQ at three random
    128-row blocks, the empty one and the last; dK and dV at three random
    128-key workgroups, the one holding the empty key block and the last,
    against the oracle's gradients there; the empty blocks' gradients are
    exactly 0."""
    w = WORKLOADS["patch_3mp"]
    q, k, v = (t[:, :1].contiguous() for t in make_inputs(w))
    do = make_inputs(Workload("do", 1, 1, w.N, 64, "bf16", 1.0, w.scale, causal, w.seed + 61, ""))[0]
    m = random_mask(w.N, 0.5, seed=6300)
    m[40] = 0          # query rows 5,120 .. 5,247 see no key
    m[:, 90] = 0       # keys 5,760 .. 5,823 are seen by no query
    print(f"[case] 3 MP block-sparse causal={causal}", flush=True)
    dq, dk, dv = run(q, k, v, do, causal, m)
    rows = np.unique(np.concatenate([block_rows(w.N, 3, seed=85, rows_per_block=128), np.arange(5120, 5248)]))
    keys = np.unique(np.concatenate([block_rows(w.N, 3, seed=86, rows_per_block=128), np.arange(5760, 5888)]))
    bm = (m, 128, 64)
    ref = attention_backward_sampled(to_f64(q), to_f64(k), to_f64(v), to_f64(do), w.scale, causal, rows, keys,
                                     block_mask=bm)
    mags = grad_magnitudes_sampled(q, k, v, do, w.scale, causal, rows, keys, block_mask=bm)
    got = (dq[:, :, rows], dk[:, :, keys], dv[:, :, keys])
    for name, g, r, mg in zip(("dQ", "dK", "dV"), got, ref, mags):
        assert_grad_within(f"{name} 3 MP block-sparse causal={causal}", g, r, mg)
    assert not dq[:, :, 5120:5248].float().any(), "a query block with no key block has dQ = 0"
    assert not dk[:, :, 5760:5824].float().any() and not dv[:, :, 5760:5824].float().any(), \
        "a key block no query sees has dK = dV = 0"
