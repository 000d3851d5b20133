"""Key-padding masks on the GPU (attn_fwd_masked, attn_fwd_fp32_masked)
against the fp64 oracle.

The mask is the per-key additive bias of the Qiita page on the patch layer
(sections 4 and 6): 0 for a key that takes part, -inf for a padded key, the
same for every query of a batch entry.  Two forms: a per-entry valid length
(key j takes part iff j < key_len[b]) and a mask [B, N], one byte per key,
packed to 32 keys per word by attn_pack_key_mask.  A row that
sees no key gets O = 0 and LSE = -inf exactly (the empty sum; the oracle
follows the same reading), so such rows are compared exactly and the others
to the usual bars.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import exact_attention_29_amd as ea
from oracle import attention as oracle_attention
from tests.parity import BF16, FP32, assert_within, errors
from workloads import Workload, make_inputs, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def check(q, k, v, o, lse, scale, causal, key_valid, bar, what):
    o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), scale, causal=causal,
                                      key_valid=key_valid)
    o_h, lse_h = to_f64(o), to_f64(lse)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_h), empty), f"{what}: empty rows differ"
    assert np.all(o_h[empty] == 0.0), f"{what}: an empty row has O != 0"
    keep = ~empty
    if keep.any():
        err = errors(o_h[keep], lse_h[keep], o_ref[keep], lse_ref[keep])
        assert_within(err, bar, what)
    return int(empty.sum())


def run(q, k, v, scale, causal, key_len=None, key_valid=None):
    kl = None if key_len is None else torch.tensor(key_len, dtype=torch.int32, device=DEV)
    kv = None if key_valid is None else torch.from_numpy(np.asarray(key_valid, dtype=bool)).to(DEV)
    o, lse = ea.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal,
                        key_len=kl, key_valid=kv)
    torch.cuda.synchronize()
    return o, lse


def inputs(B, H, N, dtype, seed, sigma=1.0):
    w = Workload("mask", B, H, N, 64, dtype, sigma, 0.125, False, seed, "mask test")
    return make_inputs(w)


LENGTHS = [512, 300, 1, 0, 257, 64, 33, 511, 480, 448]


@pytest.mark.parametrize("causal", [False, True])
def test_valid_length_bf16(causal):
    """Right padding by length on a BERT-sized batch: full, ragged, one key,
    none (every row empty), one tile, one key past a tile, all but one, and
    lengths ending on a half tile and on a whole tile."""
    B, H, N = len(LENGTHS), 4, 512
    q, k, v = inputs(B, H, N, "bf16", seed=700 + causal)
    o, lse = run(q, k, v, 0.125, causal, key_len=LENGTHS)
    valid = np.arange(N)[None, :] < np.array(LENGTHS)[:, None]
    empty = check(q, k, v, o, lse, 0.125, causal, valid, BF16, f"key_len causal={causal}")
    assert empty >= H * N  # the entry with length 0


def test_valid_length_out_of_range_is_clamped():
    B, H, N = 3, 2, 200
    q, k, v = inputs(B, H, N, "bf16", seed=710)
    o, lse = run(q, k, v, 0.125, False, key_len=[-5, 10_000, 199])
    valid = np.arange(N)[None, :] < np.clip([-5, 10_000, 199], 0, N)[:, None]
    check(q, k, v, o, lse, 0.125, False, valid, BF16, "clamped key_len")


def test_valid_length_all_keys_matches_unmasked_bitwise():
    """key_len = N changes nothing: the masked entry point gives the very
    same bits as attn_fwd."""
    B, H, N = 2, 3, 1000
    q, k, v = (t.to(DEV) for t in inputs(B, H, N, "bf16", seed=720))
    o0, l0 = ea.forward(q, k, v, scale=0.125)
    o1, l1 = ea.forward(q, k, v, scale=0.125, key_len=torch.full((B,), N, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("n", [64, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_byte_mask_bf16(n, causal):
    """Random padding patterns (30% of keys hidden), one batch entry with no
    key at all, one whose first 64 keys are hidden (the first tile sees
    nothing), and a key-length cut on top for the last entry."""
    B, H = 4, 3
    rng = np.random.default_rng(730 + n + causal)
    valid = rng.random((B, n)) >= 0.3
    valid[1] = False
    valid[2, :64] = False
    q, k, v = inputs(B, H, n, "bf16", seed=731 + n)
    lens = [n, n, n, max(1, n // 3)]
    o, lse = run(q, k, v, 0.125, causal, key_len=lens, key_valid=valid)
    both = valid & (np.arange(n)[None, :] < np.array(lens)[:, None])
    check(q, k, v, o, lse, 0.125, causal, both, BF16, f"byte mask n={n} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_byte_mask_all_true_matches_unmasked(causal):
    B, H, N = 2, 2, 700
    q, k, v = inputs(B, H, N, "bf16", seed=740 + causal)
    o, lse = run(q, k, v, 0.125, causal, key_valid=np.ones((B, N), dtype=bool))
    check(q, k, v, o, lse, 0.125, causal, None, BF16, "all-true byte mask")


@pytest.mark.parametrize("causal", [False, True])
def test_masks_fp32(causal):
    B, H, N = 3, 2, 150
    rng = np.random.default_rng(750 + causal)
    valid = rng.random((B, N)) >= 0.4
    valid[0] = False
    q, k, v = inputs(B, H, N, "fp32", seed=751)
    lens = [N, 77, 5]
    o, lse = run(q, k, v, 0.125, causal, key_len=lens, key_valid=valid)
    both = valid & (np.arange(N)[None, :] < np.array(lens)[:, None])
    check(q, k, v, o, lse, 0.125, causal, both, FP32, f"fp32 masks causal={causal}")


@pytest.mark.parametrize("n", [1, 31, 32, 33, 300, 1000])
def test_pack_key_mask_bits(n):
    """attn_pack_key_mask: bit j%32 of word j/32 = key j valid, bits past N zero
    (compared with numpy's little-endian packbits, exact)."""
    rng = np.random.default_rng(760 + n)
    valid = rng.random((3, n)) >= 0.5
    valid[1] = True
    for dtype in (torch.bool, torch.uint8):
        t = torch.from_numpy(valid).to(dtype).to(DEV)
        if dtype == torch.uint8:
            t = t * torch.randint(1, 255, t.shape, dtype=torch.uint8, device=DEV)  # any non-zero byte
        bits = ea.pack_key_mask(t)
        torch.cuda.synchronize()
        words = (n + 31) // 32
        pad = np.zeros((3, words * 32), dtype=bool)
        pad[:, :n] = valid
        ref = np.packbits(pad.reshape(3, words, 4, 8), axis=-1, bitorder="little").reshape(3, words * 4)
        ref = ref.view(np.uint32).reshape(3, words)
        assert np.array_equal(bits.cpu().numpy().view(np.uint32), ref)


def test_packed_bits_given_directly():
    B, H, N = 2, 2, 129
    rng = np.random.default_rng(770)
    valid = rng.random((B, N)) >= 0.25
    q, k, v = inputs(B, H, N, "bf16", seed=771)
    bits = ea.pack_key_mask(torch.from_numpy(valid).to(DEV))
    o, lse = ea.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=0.125, key_bits=bits)
    torch.cuda.synchronize()
    check(q, k, v, o, lse, 0.125, False, valid, BF16, "key_bits")


def test_page_mask_polarity_example_on_the_gpu():
    """The Qiita page's worked example (section 6): q = k = v from
    torch.manual_seed(0); torch.randn(1, 2, 4, 8), key 3 padded, scale
    1/sqrt(8).  The head size is padded with zeros to 64 (zero features add
    nothing to any score or output).  Keeping keys 0..2 must match the
    oracle, and attending only key 3 (the un-inverted boolean mask) must
    differ from it by the printed 3.46."""
    with open(os.path.join(GOLDEN, "mask_polarity_example.json")) as f:
        g = json.load(f)
    x = torch.randn(1, 2, 4, 8, generator=torch.Generator().manual_seed(0))
    xp = torch.zeros(1, 2, 4, 64)
    xp[..., :8] = x
    scale = 1.0 / math.sqrt(8)
    keep = np.array([[True, True, True, False]])
    o_keep, l_keep = run(xp, xp, xp, scale, False, key_valid=keep)
    o_asis, _ = run(xp, xp, xp, scale, False, key_valid=~keep)
    check(xp, xp, xp, o_keep, l_keep, scale, False, keep, FP32, "page example")
    got = round(float((o_asis - o_keep).abs().max()), g["printed_decimals"])
    assert got == g["cases"]["boolean_mask_as_is_attends_only_key_3"], got


@pytest.mark.parametrize("n", [64 * t + r for t in range(1, 21, 3) for r in (0, 37)] +
                         [64 * 13, 64 * 19 + 5, 64 * 5 + 32, 64 * 12 + 32])
def test_key_mask_ring_lengths(n):
    """The key-mask kernel over key-tile counts 1 .. 19 (the 8-wave kernel's
    paired ring: partial turns and general tails of every parity, last tiles
    of one and two whole half tiles, which drain with the mask words read
    ahead), with a random tenth of the keys hidden and key 0 kept."""
    rng = np.random.default_rng(7000 + n)
    valid = rng.random((2, n)) > 0.1
    valid[:, 0] = True
    q, k, v = inputs(2, 2, n, "bf16", 7100 + n)
    o, lse = run(q, k, v, 0.125, False, key_valid=valid)
    check(q, k, v, o, lse, 0.125, False, valid, BF16, f"mask ring N={n}")


@pytest.mark.parametrize("n", [64 * t + r for t in (3, 6, 10, 17) for r in (0, 32, 45)])
def test_causal_key_mask_ring_lengths(n):
    """Causal rows with both key-mask forms over several tile counts and
    ends (whole tile, one half tile, ragged): each wave's last visible half
    tile drains in the pipeline with the diagonal or the valid length as a
    per-row limit, the mask words on top.  Entry 1's valid length ends
    inside the sequence, so rows past it are limited by the length instead
    of the diagonal; entry 2's ends on a half-tile boundary."""
    B, H = 3, 2
    rng = np.random.default_rng(7300 + n)
    valid = rng.random((B, n)) > 0.1
    valid[:, 0] = True
    lens = [n, max(1, (2 * n) // 3), max(32, 32 * (n // 64))]
    q, k, v = inputs(B, H, n, "bf16", 7310 + n)
    o, lse = run(q, k, v, 0.125, True, key_len=lens, key_valid=valid)
    both = valid & (np.arange(n)[None, :] < np.array(lens)[:, None])
    check(q, k, v, o, lse, 0.125, True, both, BF16, f"causal mask ring N={n}")


@pytest.mark.parametrize("B, H", [(3, 21), (4, 16)])
def test_key_mask_wave_count_threshold(B, H):
    """The key-mask kernel on both sides of the 4-wave / 8-wave choice
    (N = 1000: 63 heads below it, 64 at it), a random tenth of keys hidden."""
    rng = np.random.default_rng(7300 + B)
    valid = rng.random((B, 1000)) > 0.1
    valid[:, 0] = True
    q, k, v = inputs(B, H, 1000, "bf16", 7400 + B)
    o, lse = run(q, k, v, 0.125, False, key_valid=valid)
    check(q, k, v, o, lse, 0.125, False, valid, BF16, f"mask threshold {B}x{H}")



@pytest.mark.parametrize("causal", [False, True])
def test_patch_3mp_random_key_mask(causal):
    """The 3 MP patch workload (B=1 plus a second entry, H=16, N=11,616) with
    real padding: entry 0 has a random ~10% of keys masked, entry 1 a valid
    length of 10,000 and the same kind of random mask; both masks go to the
    masked kernel at once.  Compared with the oracle on eight random 256-row
    blocks per head (every row offset of a workgroup) plus the last block."""
    from workloads import WORKLOADS, block_rows
    base = WORKLOADS["patch_3mp"]
    w = Workload("patch_3mp_masked", 2, base.H, base.N, 64, "bf16", base.sigma, base.scale, causal,
                 base.seed + 10, "")
    q, k, v = make_inputs(w)
    rng = np.random.default_rng(77)
    valid = rng.random((2, w.N)) >= 0.10
    key_len = [w.N, 10000]
    print(f"[case] 3 MP masked causal={causal}: {int((~valid).sum())} keys masked, key_len={key_len}", flush=True)
    o, lse = run(q, k, v, w.scale, causal, key_len=key_len, key_valid=valid)
    eff = valid & (np.arange(w.N)[None, :] < np.array(key_len)[:, None])
    rows = block_rows(w.N, 8, seed=78)
    o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), w.scale, causal=causal,
                                      key_valid=eff, rows=rows)
    o_h, lse_h = to_f64(o)[:, :, rows], to_f64(lse)[:, :, rows]
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_h), empty), "empty rows differ"
    keep = ~empty
    err = errors(o_h[keep], lse_h[keep], o_ref[keep], lse_ref[keep])
    assert_within(err, BF16, "3 MP masked")
    print(f"[ok] 3 MP masked causal={causal} rows/head={len(rows)} {err}", flush=True)
