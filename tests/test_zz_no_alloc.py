"""attn_bwd_noalloc through the C ABI against attn_bwd.

attn_bwd_noalloc is attn_bwd with its workspace in the library's static
device scratch instead of a caller-provided buffer.  Both run the same
kernels, so the gradients must be bit-identical.  Checked on calls in a row
that reuse the scratch: the largest size the scratch holds, then smaller
inputs (causal and not), with no device memory allocated by the calls, and
a call past the limit refused with ATTN_E_SCRATCH before anything runs.
The first call on a device looks up the array's device address, and the
runtime then places the array (16 MiB plus its rounding) on that device:
that set-up call is made, and checked, before memory is watched.
"""

import pytest
import torch

import exact_attention_29_amd as ea
from workloads import Workload, make_device_normal, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load_library()
    yield
    torch.cuda.synchronize()


def _inputs(B, H, N, seed, device_draw=False):
    if device_draw:
        q, k, v, do = (make_device_normal((B, H, N, 64), seed + i, DEV) for i in range(4))
    else:
        w = Workload("noalloc", B, H, N, 64, "bf16", 1.0, 0.125, False, seed, "")
        q, k, v = (t.to(DEV) for t in make_inputs(w))
        do = make_inputs(Workload("noalloc_do", B, H, N, 64, "bf16", 1.0, 0.125, False, seed + 1, ""))[0].to(DEV)
    return q, k, v, do


def _ptrs(*ts):
    return [t.data_ptr() for t in ts]


def _with_workspace(q, k, v, o, lse, do, causal):
    B, H, N, d = q.shape
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(ea.attn_bwd_workspace_size(B, H, N), dtype=torch.uint8, device=DEV)
    ea.attn_bwd(*_ptrs(q, k, v, o, lse, do, dq, dk, dv, ws), B, H, N, d, 0.125, causal,
                torch.cuda.current_stream().cuda_stream)
    return dq, dk, dv


def test_noalloc_matches_attn_bwd_on_calls_in_a_row():
    cases = [(1, 2, 200, False, False),      # set-up: the first call on this device
             (1, 16, 131072, False, True),   # the largest size the 16 MiB scratch holds
             (2, 4, 1000, False, False),     # then smaller inputs reuse it
             (1, 3, 300, True, False)]
    for i, (B, H, N, causal, device_draw) in enumerate(cases):
        print(f"[case] noalloc call {i}: B={B} H={H} N={N} causal={causal}", flush=True)
        assert ea.attn_bwd_workspace_size(B, H, N) <= ea.BWD_NOALLOC_SCRATCH_BYTES
        q, k, v, do = _inputs(B, H, N, 700 + 10 * i, device_draw)
        o, lse = ea.forward(q, k, v, scale=0.125, causal=causal)
        dq, dk, dv = (torch.full_like(q, 7.0) for _ in range(3))
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        free0 = torch.cuda.mem_get_info()[0]
        ea.attn_bwd_noalloc(*_ptrs(q, k, v, o, lse, do, dq, dk, dv), B, H, N, 64, 0.125, causal,
                            torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.cuda.max_memory_allocated() == base, "the call allocated through torch"
        if i > 0:
            assert torch.cuda.mem_get_info()[0] == free0, "device memory changed during the call"
        ref = _with_workspace(q, k, v, o, lse, do, causal)
        torch.cuda.synchronize()
        for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            assert bool(torch.isfinite(got.float()).all()), f"call {i}: {name} not finite"
            assert torch.equal(got, want), f"call {i}: {name} differs from attn_bwd's"
        del q, k, v, do, o, lse, dq, dk, dv, ref
        torch.cuda.empty_cache()


def test_noalloc_refuses_sizes_past_the_scratch():
    B, H, N = 1, 16, 131073  # one row past the limit
    assert ea.attn_bwd_workspace_size(B, H, N) > ea.BWD_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(64, dtype=torch.bfloat16, device=DEV)  # never read: refused before any launch
    dq = torch.full((64,), 3.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(16, device=DEV)
    with pytest.raises(ea.AttnError) as e:
        ea.attn_bwd_noalloc(*_ptrs(q, q, q, q, lse, q, dq, dq, dq), B, H, N, 64, 0.125, False,
                            torch.cuda.current_stream().cuda_stream)
    assert e.value.code == ea.ATTN_E_SCRATCH
    torch.cuda.synchronize()
    assert bool((dq == 3.0).all())
