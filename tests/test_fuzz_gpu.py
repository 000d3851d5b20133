"""Seeded random combinations of the forward's and backward's features on the
GPU against the fp64 oracle: shapes (lengths near and between tile
boundaries), causal or not, both key-mask forms (with entries that hide every
key), packed strided views, fp32 I/O, negative and unusual scales, random
block-sparse masks, and the backward.  Each
feature has its own tests; these check that they combine.  The cases are
drawn once from a fixed seed, so every run sees the same list.  Inputs are
standard normal and scales reach 1 (eight times the workloads'), so rows
can be far sharper: the bf16 max bar is the rounding bound of bf16_bar_for.
"""

import numpy as np
import pytest
import torch

import exact_attention_29_amd as ea
from oracle import attention, attention_backward
from tests.parity import BF16, FP32, assert_grad_within, assert_within, bf16_bar_for, errors, grad_magnitudes
from workloads import Workload, make_inputs, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _length(rng):
    if rng.random() < 0.5:  # near a multiple of 32, 64, 128 or 256
        base = int(rng.choice([32, 64, 128, 256])) * int(rng.integers(1, 9))
        return max(1, base + int(rng.integers(-2, 3)))
    return int(rng.integers(1, 2100))


def _forward_cases(count=96, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        dtype = "fp32" if rng.random() < 0.15 else "bf16"
        cases.append(dict(
            i=i, B=int(rng.integers(1, 4)), H=int(rng.integers(1, 6)), N=_length(rng),
            causal=bool(rng.random() < 0.5),
            mask=str(rng.choice(["none", "len", "valid"])),
            packed=bool(dtype == "bf16" and rng.random() < 0.3),
            dtype=dtype,
            scale=float(0.125 if rng.random() < 0.6 else rng.uniform(-0.5, 1.0)),
            seed=int(rng.integers(0, 2**31))))
    return cases


FORWARD_CASES = _forward_cases()


def _mask(case, rng):
    B, N = case["B"], case["N"]
    if case["mask"] == "len":
        lens = rng.integers(0, N + 1, size=B)
        if B > 1 and rng.random() < 0.3:
            lens[0] = 0  # an entry that hides every key
        valid = np.arange(N)[None, :] < lens[:, None]
        return dict(key_len=torch.tensor(lens, dtype=torch.int32, device=DEV)), valid
    if case["mask"] == "valid":
        valid = rng.random((B, N)) < rng.uniform(0.3, 1.0)
        if B > 1 and rng.random() < 0.3:
            valid[-1] = False
        return dict(key_valid=torch.from_numpy(valid).to(DEV)), valid
    return {}, None


@pytest.mark.parametrize("case", FORWARD_CASES, ids=lambda c: "c%02d_%s_N%d%s%s_%s_%s" % (
    c["i"], c["dtype"], c["N"], "_causal" if c["causal"] else "", "_packed" if c["packed"] else "",
    c["mask"], "B%dH%d" % (c["B"], c["H"])))
def test_random_forward(case):
    B, H, N = case["B"], case["H"], case["N"]
    print(f"[fuzz] {case}", flush=True)
    w = Workload("fuzz", B, H, N, 64, case["dtype"], 1.0, case["scale"], case["causal"], case["seed"], "")
    q, k, v = make_inputs(w)
    rng = np.random.default_rng(case["seed"])
    kwargs, valid = _mask(case, rng)
    if case["packed"]:
        # the head views of one packed [B, N, 3*H*64] projection holding q, k, v
        x = torch.cat([t.transpose(1, 2).reshape(B, N, H * 64) for t in (q, k, v)], dim=-1).to(DEV)
        qd, kd, vd = (t.view(B, N, H, 64).transpose(1, 2) for t in x.chunk(3, dim=-1))
    else:
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o, lse = ea.forward(qd, kd, vd, scale=case["scale"], causal=case["causal"], **kwargs)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention(to_f64(q), to_f64(k), to_f64(v), case["scale"], causal=case["causal"],
                               key_valid=valid)
    o_h, lse_h = to_f64(o.contiguous()), to_f64(lse)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_h), empty), "rows that see no key differ"
    assert np.all(o_h[empty] == 0.0), "a row that sees no key has O != 0"
    keep = ~empty
    if keep.any():
        bar = FP32 if case["dtype"] == "fp32" else bf16_bar_for(float(v.abs().max()), float(np.abs(o_ref[keep]).max()))
        assert_within(errors(o_h[keep], lse_h[keep], o_ref[keep], lse_ref[keep]), bar, f"case {case['i']}")


def _backward_cases(count=12, seed=4048):
    rng = np.random.default_rng(seed)
    return [dict(i=i, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), N=_length(rng) // 2 + 1,
                 causal=bool(rng.random() < 0.5),
                 scale=float(0.125 if rng.random() < 0.6 else rng.uniform(-0.4, 0.6)),
                 seed=int(rng.integers(0, 2**31))) for i in range(count)]


@pytest.mark.parametrize("case", _backward_cases(), ids=lambda c: "b%02d_N%d%s_B%dH%d" % (
    c["i"], c["N"], "_causal" if c["causal"] else "", c["B"], c["H"]))
def test_random_backward(case):
    B, H, N = case["B"], case["H"], case["N"]
    print(f"[fuzz] {case}", flush=True)
    w = Workload("fuzz_bwd", B, H, N, 64, "bf16", 1.0, case["scale"], case["causal"], case["seed"], "")
    q, k, v = make_inputs(w)
    do = make_inputs(Workload("fuzz_do", B, H, N, 64, "bf16", 1.0, case["scale"], case["causal"],
                              case["seed"] + 1, ""))[0]
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = ea.forward(qd, kd, vd, scale=case["scale"], causal=case["causal"])
    grads = ea.backward(qd, kd, vd, o, lse, dod, scale=case["scale"], causal=case["causal"])
    torch.cuda.synchronize()
    ref = attention_backward(to_f64(q), to_f64(k), to_f64(v), to_f64(do), case["scale"], causal=case["causal"])
    mags = grad_magnitudes(q, k, v, do, case["scale"], case["causal"])
    for name, g, r, m in zip(("dQ", "dK", "dV"), grads, ref, mags):
        assert_grad_within(f"{name} case {case['i']}", g, r, m)


def _sparse_cases(count=12, seed=6072):
    rng = np.random.default_rng(seed)
    return [dict(i=i, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), N=_length(rng),
                 causal=bool(rng.random() < 0.5), density=float(rng.uniform(0.05, 1.0)),
                 scale=float(0.125 if rng.random() < 0.7 else rng.uniform(-0.5, 1.0)),
                 seed=int(rng.integers(0, 2**31))) for i in range(count)]


@pytest.mark.parametrize("case", _sparse_cases(), ids=lambda c: "s%02d_N%d%s_d%.2f" % (
    c["i"], c["N"], "_causal" if c["causal"] else "", c["density"]))
def test_random_block_sparse(case):
    """Random block masks (128-query by 64-key blocks) at random density,
    rows whose blocks are all unset included."""
    B, H, N = case["B"], case["H"], case["N"]
    print(f"[fuzz] {case}", flush=True)
    w = Workload("fuzz_sparse", B, H, N, 64, "bf16", 1.0, case["scale"], case["causal"], case["seed"], "")
    q, k, v = make_inputs(w)
    rng = np.random.default_rng(case["seed"])
    nbq, nbk = -(-N // ea.SPARSE_BLOCK_Q), -(-N // ea.SPARSE_BLOCK_K)
    m = rng.random((nbq, nbk)) < case["density"]
    o, lse = ea.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=case["scale"], causal=case["causal"],
                        block_mask=torch.from_numpy(m).to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = attention(to_f64(q), to_f64(k), to_f64(v), case["scale"], causal=case["causal"],
                               block_mask=(m, ea.SPARSE_BLOCK_Q, ea.SPARSE_BLOCK_K))
    o_h, lse_h = to_f64(o), to_f64(lse)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_h), empty), "rows that see no key differ"
    assert np.all(o_h[empty] == 0.0), "a row that sees no key has O != 0"
    keep = ~empty
    if keep.any():
        bar = bf16_bar_for(float(v.abs().max()), float(np.abs(o_ref[keep]).max()))
        assert_within(errors(o_h[keep], lse_h[keep], o_ref[keep], lse_ref[keep]), bar, f"case {case['i']}")
