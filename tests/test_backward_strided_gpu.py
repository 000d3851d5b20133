"""Strided backward on the GPU (attn_bwd_strided).

Training through the patch layer of the Qiita page (section 4: one packed
input projection [B, N, 3*H*d], split into q, k, v and viewed per head)
needs the gradient of that projection: dq, dk, dv are written straight into
head views of one packed gradient buffer, and q, k, v, o, dout are read in
place.  The strided kernels form each row's address from its strides and
otherwise do the same arithmetic, so every gradient must equal, bit for
bit, the contiguous backward on contiguous copies of the same values
(which the other backward tests compare with the fp64 oracle); one case is
also compared with the oracle directly.
"""

import numpy as np
import pytest
import torch

import exact_attention_29_amd as ea
from oracle import attention_backward
from tests.parity import assert_grad_within, grad_magnitudes
from workloads import WORKLOADS, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def packed(B, N, H, seed, sigma=1.0):
    """A [B, N, 3*H*64] bf16 projection output and its q, k, v head views."""
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(B, N, 3 * H * 64, generator=g) * sigma).to(torch.bfloat16).to(DEV)
    return x, tuple(t.view(B, N, H, 64).transpose(1, 2) for t in x.chunk(3, dim=-1))


def token_major(B, N, H, seed):
    """A [B, N, H, 64] bf16 tensor (what the output projection's gradient
    gives) as its [B, H, N, 64] view."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn(B, N, H, 64, generator=g).to(torch.bfloat16).to(DEV).transpose(1, 2)


def run_both(q, k, v, dout, causal, masks, o_view=None):
    """Forward on the views, then the strided backward (q, k, v, o, dout as
    views, dq, dk, dv into a packed gradient buffer) and the contiguous
    backward on copies; returns both gradient triples."""
    B, H, N, _ = q.shape
    o, lse = ea.forward(q, k, v, scale=0.125, causal=causal, out=o_view, **masks)
    gx = torch.full((B, N, 3 * H * 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    dq, dk, dv = (t.view(B, N, H, 64).transpose(1, 2) for t in gx.chunk(3, dim=-1))
    ea.backward(q, k, v, o, lse, dout, scale=0.125, causal=causal, dq=dq, dk=dk, dv=dv, **masks)
    qc, kc, vc, oc, dc = (t.contiguous() for t in (q, k, v, o, dout))
    ref = ea.backward(qc, kc, vc, oc, lse, dc, scale=0.125, causal=causal, **masks)
    torch.cuda.synchronize()
    return (dq, dk, dv), ref


@pytest.mark.parametrize("n", [1, 65, 300, 1000, 2100])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_gradient_matches_contiguous_bitwise(n, causal):
    B, H = 2, 3
    _, (q, k, v) = packed(B, n, H, seed=900 + n)
    dout = token_major(B, n, H, seed=950 + n)
    print(f"[case] packed n={n} causal={causal}", flush=True)
    got, ref = run_both(q, k, v, dout, causal, {})
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(g, r), f"{name} differs from the contiguous backward (n={n}, causal={causal})"


@pytest.mark.parametrize("mask", ["len", "bits"])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_gradient_with_key_masks(mask, causal):
    B, H, n = 3, 2, 777
    _, (q, k, v) = packed(B, n, H, seed=1000)
    dout = token_major(B, n, H, seed=1001)
    if mask == "len":
        masks = {"key_len": torch.tensor([777, 300, 0], dtype=torch.int32, device=DEV)}
    else:
        valid = np.random.default_rng(1002).random((B, n)) < 0.6
        valid[2] = False
        masks = {"key_valid": torch.tensor(valid, device=DEV)}
    print(f"[case] packed {mask} causal={causal}", flush=True)
    got, ref = run_both(q, k, v, dout, causal, masks)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(g, r), f"{name} differs from the contiguous backward ({mask}, causal={causal})"


def test_token_major_output_and_shared_kv():
    """o written token-major by the forward and read so by the backward; K
    and V one [B, N, 64] tensor shared by every head (head stride 0), so
    dK and dV are per-head gradients of that shared tensor."""
    B, H, n = 2, 4, 513
    g = torch.Generator().manual_seed(1100)
    q = torch.randn(B, H, n, 64, generator=g).to(torch.bfloat16).to(DEV)
    kv = torch.randn(B, n, 2, 64, generator=g).to(torch.bfloat16).to(DEV)
    k = kv[:, :, 0].unsqueeze(1).expand(B, H, n, 64)
    v = kv[:, :, 1].unsqueeze(1).expand(B, H, n, 64)
    assert k.stride(1) == 0
    o_tok = torch.empty(B, n, H, 64, dtype=torch.bfloat16, device=DEV)
    dout = token_major(B, n, H, seed=1101)
    got, ref = run_both(q, k, v, dout, False, {}, o_view=o_tok.transpose(1, 2))
    for name, gr, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(gr, r), f"{name} differs from the contiguous backward"


def test_packed_gradient_against_oracle():
    """The packed case once against the fp64 oracle directly."""
    B, H, n = 1, 2, 600
    _, (q, k, v) = packed(B, n, H, seed=1200)
    dout = token_major(B, n, H, seed=1201)
    got, _ = run_both(q, k, v, dout, True, {})
    qc, kc, vc, dc = (t.contiguous() for t in (q, k, v, dout))
    ref = attention_backward(to_f64(qc), to_f64(kc), to_f64(vc), to_f64(dc), 0.125, causal=True)
    mags = grad_magnitudes(qc, kc, vc, dc, 0.125, True)
    for name, g, r, m in zip(("dQ", "dK", "dV"), got, ref, mags):
        assert_grad_within(f"{name} packed", g.contiguous(), r, m)


def test_packed_gradient_patch_3mp_bitwise():
    """The 3 MP patch shape (N = 11,616, 16 heads) from one packed
    projection: the strided backward equals the contiguous one bit for bit."""
    w = WORKLOADS["patch_3mp"]
    _, (q, k, v) = packed(1, w.N, w.H, seed=1300, sigma=0.5)
    dout = token_major(1, w.N, w.H, seed=1301)
    print("[case] packed 3 MP", flush=True)
    got, ref = run_both(q, k, v, dout, False, {})
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(g, r), f"{name} differs from the contiguous backward at 3 MP"


def test_strided_binding_checks():
    """A block mask with strided tensors, or outputs of the wrong shape, are
    refused before anything is launched."""
    B, H, n = 1, 2, 200
    _, (q, k, v) = packed(B, n, H, seed=1400)
    o, lse = ea.forward(q, k, v)
    dout = token_major(B, n, H, seed=1401)
    m = torch.ones((2, 4), dtype=torch.bool, device=DEV)
    with pytest.raises(ValueError):
        ea.backward(q, k, v, o, lse, dout, block_mask=m)
    with pytest.raises(ValueError):
        ea.backward(q, k, v, o, lse, dout, dq=torch.empty(B, H, n, 32, dtype=torch.bfloat16, device=DEV))
