"""Strided inputs on the GPU (attn_fwd_strided) against the fp64 oracle.

The Qiita page on the patch layer, section 4, builds q, k, v from one packed
input projection [B, N, 3*H*d]: split in three, viewed per head and
transposed to [B, H, N, d].  attn_fwd_strided reads those views in place.
The oracle gets contiguous copies of the same values.
"""

import numpy as np
import pytest
import torch

import exact_attention_29_amd as ea
from oracle import attention as oracle_attention
from tests.parity import BF16, assert_within, errors
from workloads import WORKLOADS, Workload, block_rows, make_inputs, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def packed_views(B, N, H, seed, sigma=1.0):
    """One [B, N, 3*H*64] bf16 projection output and its q, k, v head views."""
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(B, N, 3 * H * 64, generator=g) * sigma).to(torch.bfloat16).to(DEV)
    q, k, v = (t.view(B, N, H, 64).transpose(1, 2) for t in x.chunk(3, dim=-1))
    return x, q, k, v


def compare(q, k, v, o, lse, scale, causal, what, rows=None, key_valid=None):
    qc, kc, vc = (to_f64(t.contiguous()) for t in (q, k, v))
    o_ref, l_ref = oracle_attention(qc, kc, vc, scale, causal=causal, rows=rows, key_valid=key_valid)
    o_h, l_h = to_f64(o.contiguous()), to_f64(lse)
    if rows is not None:
        o_h, l_h = o_h[:, :, rows], l_h[:, :, rows]
    assert_within(errors(o_h, l_h, o_ref, l_ref), BF16, what)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_projection_views(causal):
    B, N, H = 2, 1000, 4
    _, q, k, v = packed_views(B, N, H, seed=800 + causal)
    assert not q.is_contiguous() and q.stride() == (N * 3 * H * 64, 64, 3 * H * 64, 1)
    o, lse = ea.forward(q, k, v, scale=0.125, causal=causal)
    torch.cuda.synchronize()
    compare(q, k, v, o, lse, 0.125, causal, f"packed views causal={causal}")


def test_strided_output_in_token_major_layout():
    """o written as [B, N, H, d] (what the output projection reads)."""
    B, N, H = 2, 333, 3
    _, q, k, v = packed_views(B, N, H, seed=810)
    o_tok = torch.empty(B, N, H, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = ea.forward(q, k, v, scale=0.125, out=o_tok.transpose(1, 2))
    torch.cuda.synchronize()
    compare(q, k, v, o_tok.transpose(1, 2), lse, 0.125, False, "token-major output")


def test_kv_shared_by_heads():
    """Head stride 0 for K and V: every head reads the same keys and values."""
    B, H, N = 2, 4, 500
    w = Workload("mqa", B, 1, N, 64, "bf16", 1.0, 0.125, False, 820, "")
    q_all = make_inputs(Workload("mqa_q", B, H, N, 64, "bf16", 1.0, 0.125, False, 821, ""))[0].to(DEV)
    _, k1, v1 = (t.to(DEV) for t in make_inputs(w))
    k, v = k1.expand(B, H, N, 64), v1.expand(B, H, N, 64)
    assert k.stride(1) == 0
    o, lse = ea.forward(q_all, k, v, scale=0.125)
    torch.cuda.synchronize()
    compare(q_all, k, v, o, lse, 0.125, False, "shared K/V")


def test_strided_with_padding_length():
    B, N, H = 3, 400, 2
    _, q, k, v = packed_views(B, N, H, seed=830)
    lens = [400, 130, 0]
    o, lse = ea.forward(q, k, v, scale=0.125, key_len=torch.tensor(lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    valid = np.arange(N)[None, :] < np.array(lens)[:, None]
    qc, kc, vc = (to_f64(t.contiguous()) for t in (q, k, v))
    o_ref, l_ref = oracle_attention(qc, kc, vc, 0.125, key_valid=valid)
    o_h, l_h = to_f64(o), to_f64(lse)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_h), empty) and np.all(o_h[empty] == 0.0)
    assert_within(errors(o_h[~empty], l_h[~empty], o_ref[~empty], l_ref[~empty]), BF16, "strided + key_len")


def test_patch_3mp_packed_views_match_contiguous_bitwise():
    """At the 3 MP patch shape the strided call does the same arithmetic as
    the contiguous one on copies of the same values: identical bits; and
    sampled rows match the oracle."""
    w = WORKLOADS["patch_3mp"]
    B, H, N, d = w.shape
    _, q, k, v = packed_views(B, N, H, seed=w.seed, sigma=w.sigma)
    o_s, l_s = ea.forward(q, k, v, scale=w.scale)
    o_c, l_c = ea.forward(q.contiguous(), k.contiguous(), v.contiguous(), scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_c) and torch.equal(l_s, l_c)
    compare(q, k, v, o_s, l_s, w.scale, False, "3 MP packed views", rows=block_rows(N, 4, seed=3))


def test_misaligned_stride_is_refused():
    B, N, H = 1, 64, 2
    x = torch.zeros(B, N, 3 * H * 64 + 4, dtype=torch.bfloat16, device=DEV)  # row stride 388: not a multiple of 8
    q, k, v = (x[..., i * H * 64:(i + 1) * H * 64].view(B, N, H, 64).transpose(1, 2) for i in range(3))
    with pytest.raises(ea.AttnError):
        ea.forward(q, k, v)
