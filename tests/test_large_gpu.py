"""Tensors of more than 2^31 elements (over 4 GiB of bf16 each).

B = 2 entries of H = 8,200 heads, N = 2,048 rows, d = 64: 2,149,580,800
elements per tensor.  Heads and batch entries are addressed with 64-bit
offsets, so the whole call runs; the heads whose data starts at or past
element 2^31 (byte offset 2^32 of a bf16 tensor: entry 1, heads 8,184 on)
are checked beside heads below that boundary, each against the oracle with
the bars every other parity test uses (a 32-bit offset anywhere would land
such a head on another head's random data).
"""

import gc

import numpy as np
import pytest
import torch

import exact_attention_29_amd as ea
from oracle import attention, attention_backward
from tests.parity import BF16, FP32, assert_grad_within, assert_within, errors, grad_magnitudes
from workloads import make_device_normal, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B, H, N, D = 2, 8200, 2048, 64
SCALE = 0.125
# (entry, head): the first head, one below the boundary, the first head at
# element 2^31, one past it, the last head of each entry
HEADS = [(0, 0), (0, 8199), (1, 8183), (1, 8184), (1, 8191), (1, 8199)]


def boundary_head():
    return (1 * H + 8184) * N * D


def inputs(dtype, seed):
    assert boundary_head() == 1 << 31
    torch.cuda.empty_cache()
    return tuple(make_device_normal((B, H, N, D), seed + i, DEV, dtype) for i in range(3))


def head(t, b, h):
    """Head (b, h) of a device tensor as a float64 [1, 1, N, d] array."""
    return to_f64(t[b, h][None, None])


def release():
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_forward_past_2_31_elements(causal):
    q, k, v = inputs("bf16", 9000)
    assert q.numel() > (1 << 31)
    o, lse = ea.forward(q, k, v, scale=SCALE, causal=causal)
    torch.cuda.synchronize()
    for b, h in HEADS:
        o_ref, lse_ref = attention(head(q, b, h), head(k, b, h), head(v, b, h), SCALE, causal=causal)
        err = errors(to_f64(o[b, h]), to_f64(lse[b, h]), o_ref[0, 0], lse_ref[0, 0])
        print(f"[large] forward causal={causal} head ({b},{h}): {err}", flush=True)
        assert_within(err, BF16, f"head ({b},{h})")
    del q, k, v, o, lse
    release()


def test_masked_forward_past_2_31_elements():
    q, k, v = inputs("bf16", 9100)
    key_len = torch.tensor([N, 1500], dtype=torch.int32, device=DEV)
    o, lse = ea.forward(q, k, v, scale=SCALE, key_len=key_len)
    torch.cuda.synchronize()
    for b, h in HEADS:
        valid = np.arange(N) < int(key_len[b])
        o_ref, lse_ref = attention(head(q, b, h), head(k, b, h), head(v, b, h), SCALE,
                                   key_valid=valid[None, :])
        err = errors(to_f64(o[b, h]), to_f64(lse[b, h]), o_ref[0, 0], lse_ref[0, 0])
        print(f"[large] key_len head ({b},{h}): {err}", flush=True)
        assert_within(err, BF16, f"head ({b},{h})")
    del q, k, v, o, lse
    release()


def test_backward_past_2_31_elements():
    q, k, v = inputs("bf16", 9200)
    do = make_device_normal((B, H, N, D), 9210, DEV, "bf16")
    o, lse = ea.forward(q, k, v, scale=SCALE, causal=True)
    dq, dk, dv = ea.backward(q, k, v, o, lse, do, scale=SCALE, causal=True)
    torch.cuda.synchronize()
    for b, h in HEADS:
        sl = [t[b, h][None, None] for t in (q, k, v, do)]
        rq, rk, rv = attention_backward(*(head(t, b, h) for t in (q, k, v, do)), SCALE, causal=True)
        mags = grad_magnitudes(*sl, SCALE, True)
        for name, g, r, m in zip(("dQ", "dK", "dV"), (dq, dk, dv), (rq, rk, rv), mags):
            assert_grad_within(f"{name} head ({b},{h})", g[b, h][None, None], r, m)
    del q, k, v, do, o, lse, dq, dk, dv
    release()


def test_fp32_forward_past_2_31_elements():
    q, k, v = inputs("fp32", 9300)
    o, lse = ea.forward(q, k, v, scale=SCALE, causal=False)
    torch.cuda.synchronize()
    for b, h in HEADS[2:4]:
        o_ref, lse_ref = attention(head(q, b, h), head(k, b, h), head(v, b, h), SCALE)
        err = errors(to_f64(o[b, h]), to_f64(lse[b, h]), o_ref[0, 0], lse_ref[0, 0])
        print(f"[large] fp32 head ({b},{h}): {err}", flush=True)
        assert_within(err, FP32, f"head ({b},{h})")
    del q, k, v, o, lse
    release()
