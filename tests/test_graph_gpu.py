"""The entry points under stream capture: a forward and a backward recorded
into a HIP graph (torch.cuda.CUDAGraph) and replayed several times, with
other eager work and synchronisations between the replays.  The kernels
are deterministic and launch only on the caller's stream (no memsets, no
allocation), so every replay must reproduce the eager results bit for bit.
"""

import pytest
import torch

import exact_attention_29_amd as ea
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(N, seed, causal):
    w = Workload("graph", 2, 4, N, 64, "bf16", 1.0, 0.125, causal, seed, "")
    q, k, v = (t.to(DEV) for t in make_inputs(w))
    do = make_inputs(Workload("graph_do", 2, 4, N, 64, "bf16", 1.0, 0.125, causal, seed + 1, ""))[0].to(DEV)
    return q, k, v, do


@pytest.mark.parametrize("masked", ["none", "len", "bits", "blocks"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_and_backward_replay_in_a_graph(causal, masked):
    """masked: both passes with valid key lengths (one entry cut inside a
    tile), a random key bit mask (attn_fwd_masked, attn_bwd_masked), or a
    random block mask (attn_fwd_block_sparse, attn_bwd_block_sparse)."""
    q, k, v, do = _inputs(777, 9500 + causal, causal)
    masks = {}
    if masked == "len":
        masks["key_len"] = torch.tensor([777, 300], dtype=torch.int32, device=DEV)
    elif masked == "bits":
        masks["key_bits"] = ea.pack_key_mask(torch.rand(2, 777, device=DEV) < 0.6)
    elif masked == "blocks":
        masks["block_mask"] = torch.rand(-(-777 // ea.SPARSE_BLOCK_Q), -(-777 // ea.SPARSE_BLOCK_K),
                                         device=DEV) < 0.5
    # eager results (also warms the library's per-device state up before capture)
    o_ref, lse_ref = ea.forward(q, k, v, scale=0.125, causal=causal, **masks)
    g_ref = ea.backward(q, k, v, o_ref, lse_ref, do, scale=0.125, causal=causal, **masks)
    torch.cuda.synchronize()

    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            ea.forward(q, k, v, scale=0.125, causal=causal, out=o, lse=lse, **masks)
            grads = ea.backward(q, k, v, o, lse, do, scale=0.125, causal=causal, **masks)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for replay in range(3):
        # clobber the outputs and run unrelated eager work between replays
        for t in (o, lse, *grads):
            t.fill_(float("nan") if t.dtype.is_floating_point else 0)
        torch.cuda.synchronize()
        graph.replay()
        filler = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(filler)
        assert torch.equal(o, o_ref), f"replay {replay}: O differs from the eager call"
        assert torch.equal(lse, lse_ref), f"replay {replay}: LSE differs from the eager call"
        for name, g, r in zip(("dQ", "dK", "dV"), grads, g_ref):
            assert torch.equal(g, r), f"replay {replay}: {name} differs from the eager call"


def test_masked_forward_replays_with_new_inputs():
    """A captured masked forward reads its inputs at replay time: writing new
    values into the captured input buffers changes the replayed result to
    the eager result for those values."""
    q, k, v, _ = _inputs(1000, 9600, False)
    key_len = torch.tensor([1000, 613], dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    ea.forward(q, k, v, out=o, lse=lse, key_len=key_len)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            ea.forward(q, k, v, out=o, lse=lse, key_len=key_len)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for seed in (9610, 9620):
        q2, k2, v2, _ = _inputs(1000, seed, False)
        q.copy_(q2), k.copy_(k2), v.copy_(v2)
        key_len.copy_(torch.tensor([seed % 1000 + 1, 1000], dtype=torch.int32))
        torch.cuda.synchronize()
        graph.replay()
        o_ref, lse_ref = ea.forward(q2, k2, v2, key_len=key_len.clone())
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"replay with inputs {seed}"
