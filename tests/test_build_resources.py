"""The compiler's resource report of the built library: every kernel keeps
its working set in registers and LDS.

A lambda the compiler declines to inline becomes a call with a stack frame in
scratch memory (private, per-lane HBM); at the sizes of these kernels that
slows a kernel by tens of times without changing a result, so the parity
tests cannot see it.  And a kernel that uses any scratch makes the runtime
allocate private memory for it at its first launch, which a caller that
must not allocate (attn_bwd_noalloc, graph capture) cannot have.  The bar:
no dynamic stack and no scratch anywhere, and two waves per SIMD for every
bf16 attention kernel (the occupancy the tile sizes and LDS rings are built
around).
"""

import os
import re

import pytest

from exact_attention_29_amd import build as b

MAX_SCRATCH = 0


def report():
    if not os.path.exists(b.RESOURCES):
        pytest.fail("no resource report next to the library: run the build first")
    out = {}
    for line in open(b.RESOURCES):
        name, _, fields = line.partition(": ")
        out[name] = dict(f.split("=", 1) for f in fields.split())
    return out


def test_report_lists_every_kernel():
    names = report()
    fwd = [n for n in names if "attn_fwd_bf16_kernel" in n]
    # {non-causal 8 and 4 waves, non-causal split, causal} x {key mask or not}, 2 block-sparse
    assert len(fwd) == 10, fwd
    for kind in ("attn_fwd_f32_kernel", "attn_pack_key_mask_kernel"):
        assert sum(kind in n for n in names) == 1, kind
    # causal or not; all keys, lengths, bits, blocks contiguous; all keys, lengths, bits strided
    assert sum("bwd_dkdv_kernel" in n for n in names) == 14
    assert sum("bwd_dq_kernel" in n for n in names) == 14


@pytest.mark.parametrize("name", sorted(report()) if os.path.exists(b.RESOURCES) else [])
def test_kernel_resources(name):
    r = report()[name]
    scratch = int(r["ScratchSize_[bytes/lane]"])
    assert r["Dynamic_Stack"] == "False", name
    assert scratch <= MAX_SCRATCH, f"{name}: {scratch} bytes of scratch per lane"
    if re.search(r"attn_fwd_bf16_kernel|bwd_dkdv_kernel|bwd_dq_kernel", name):
        assert int(r["Occupancy_[waves/SIMD]"]) >= 2, f"{name}: occupancy {r['Occupancy_[waves/SIMD]']}"
