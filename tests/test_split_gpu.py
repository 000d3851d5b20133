"""attn_fwd_split on the GPU: the last, partial round of 256-row query tiles
shares its tiles' keys across all CUs, and the pieces of a tile are merged
from their row maxima, row sums and unnormalised outputs (the blockwise
softmax identity of the FlashAttention reading notes, section "proposed
method", tiling).  Checked against the fp64 oracle on every row, over the
shapes that exercise each case of the decomposition:

  * a whole round and a few tiles left per XCD (two pieces per tile);
  * one tile left per XCD, cut into C pieces of one or two key tiles each
    (many-way merges);
  * tiles not a multiple of 8 (XCDs with different leftovers);
  * no whole round, long rows: every tile cut into several pieces;
  * a ragged last key tile (N not a multiple of 64) inside a piece;
  * eight seeded random shapes the library splits, with random masks and
    scales;
plus key-padding masks (pieces that see no key at all), strided head views,
NaN and infinite inputs, determinism, the arrival counters left at zero,
and replays of captured graphs.  The decomposition is deterministic (pieces
merge in a fixed order), so repeated calls give the same bits.
"""

import numpy as np
import pytest
import torch

import exact_attention_29_amd as ea
from oracle import attention as oracle_attention
from tests.parity import BF16, assert_bf16_elementwise, assert_within, errors
from workloads import Workload, make_inputs, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DEV_INDEX = 0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load_library()
    yield
    torch.cuda.synchronize()


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def count_bytes():
    """The workspace's counter block: 8 * (CUs / 8) ints, padded to 256 bytes."""
    return (8 * (cus() // 8) * 4 + 255) // 256 * 256


def splits_at(B, H, N, n_cus):
    """The library's rule for splitting a non-causal call on n_cus CUs (restated)."""
    c = n_cus // 8 if n_cus >= 16 else 1
    tiles = B * H * -(-N // 256)
    n_kt = -(-N // 64)
    per, r8 = divmod(tiles, 8)
    rounds = per // c
    rem_max = per + (1 if r8 else 0) - rounds * c
    left = tiles - 8 * rounds * c
    return (0 < rem_max < c and n_kt >= c and 2 * left <= 8 * c and (rounds >= 1 or n_kt >= 160)
            and c * c * n_kt < 2 ** 31)


def splits(B, H, N):
    return splits_at(B, H, N, cus())


def inputs(B, H, N, seed, sigma=1.0):
    return make_inputs(Workload("split", B, H, N, 64, "bf16", sigma, 0.125, False, seed, "split test"))


def run_split(q, k, v, ws=None, key_len=None, key_bits=None, layouts=None, out=None):
    """One attn_fwd_split call through the C ABI with the given (or a fresh,
    zeroed) workspace; returns O, LSE, the workspace."""
    B, H, N, d = q.shape
    if ws is None:
        ws = torch.zeros(ea.attn_fwd_split_workspace_size(B, H, N, False), dtype=torch.uint8, device=DEV)
    o = torch.empty((B, H, N, d), dtype=q.dtype, device=DEV) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    lays = layouts or (None, None, None, None)
    ea.attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                      0.125, False, *lays, 0 if key_len is None else key_len.data_ptr(),
                      0 if key_bits is None else key_bits.data_ptr(), ws.data_ptr(), ws.numel(),
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return o, lse, ws


def check(q, k, v, o, lse, what, key_valid=None):
    o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), 0.125, key_valid=key_valid)
    o_h, lse_h = to_f64(o), to_f64(lse)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_h), empty), f"{what}: empty rows differ"
    assert np.all(o_h[empty] == 0.0), f"{what}: an empty row has O != 0"
    keep = ~empty
    assert_within(errors(o_h[keep], lse_h[keep], o_ref[keep], lse_ref[keep]), BF16, what)


# (B, H, N): tiles of 256 rows = B*H*ceil(N/256); on a 256-CU part C = 32
SHAPES = [
    (2, 16, 2304),   # 288 tiles: one whole round, 4 left per XCD, 36 key tiles each
    (1, 24, 2816),   # 264 tiles: one whole round, 1 left per XCD, cut into 32 pieces
    (1, 25, 2816),   # 275 tiles: 3 left on XCDs 0-2, 2 on the others
    (1, 1, 10240),   # 40 tiles, no whole round, 160 key tiles: 5 per XCD, 6-7 pieces each
    (1, 1, 12000),   # 47 tiles (6 or 5 per XCD), ragged last key tile
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_split_matches_oracle_every_row(shape):
    B, H, N = shape
    assert splits(B, H, N), f"{shape} is expected to split on this part"
    q, k, v = inputs(B, H, N, seed=4000 + N)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o, lse, ws = run_split(qd, kd, vd)
    check(q, k, v, o, lse, f"split {shape}")
    # the partial slots were used, and the counters are back at zero
    assert int(ws[count_bytes():].count_nonzero()) > 0, "no partial result was written"
    assert int(ws[:count_bytes()].count_nonzero()) == 0, "arrival counters left non-zero"


@pytest.mark.parametrize("shape", SHAPES[:3], ids=lambda s: "x".join(map(str, s)))
def test_split_is_deterministic_and_close_to_unsplit(shape):
    B, H, N = shape
    q, k, v = (t.to(DEV) for t in inputs(B, H, N, seed=4100 + N))
    o1, l1, ws = run_split(q, k, v)
    o2, l2, _ = run_split(q, k, v, ws=ws)  # the same workspace again: counters were left at zero
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "two split calls differ"
    o0, l0 = ea.forward(q, k, v, scale=0.125, split=False)
    torch.cuda.synchronize()
    err = errors(to_f64(o1), to_f64(l1), to_f64(o0), to_f64(l0))
    assert err["o_max"] <= 2 ** -7 and err["lse_max"] <= 1e-4, err


def test_forward_uses_the_split_path_and_its_workspace():
    """forward() on a splitting shape: the same bits as attn_fwd_split with a
    fresh workspace; its cached workspace's counters end at zero."""
    B, H, N = SHAPES[0]
    q, k, v = (t.to(DEV) for t in inputs(B, H, N, seed=4200))
    o_f, l_f = ea.forward(q, k, v, scale=0.125)
    torch.cuda.synchronize()
    o_s, l_s, _ = run_split(q, k, v)
    assert torch.equal(o_f, o_s) and torch.equal(l_f, l_s)
    ws = ea.split_workspace(q.device, torch.cuda.current_stream().cuda_stream,
                            ea.attn_fwd_split_workspace_size(B, H, N, False))
    assert int(ws[:count_bytes()].count_nonzero()) == 0


def test_split_with_key_lengths():
    """Per-entry valid lengths: some pieces lie wholly past the length (they
    see no key and merge with weight 0), some rows see nothing at all."""
    B, H, N = 4, 6, 2816
    assert splits(B, H, N)
    lengths = [2816, 1, 0, 1700]
    q, k, v = inputs(B, H, N, seed=4300)
    kl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    o, lse, _ = run_split(*(t.to(DEV) for t in (q, k, v)), key_len=kl)
    valid = np.arange(N)[None, :] < np.array(lengths)[:, None]
    check(q, k, v, o, lse, "split with key_len", key_valid=valid)
    assert np.isneginf(to_f64(lse)[2]).all()


def test_split_with_random_key_mask_and_length():
    """A random ~10% key mask (packed bits) together with a length."""
    B, H, N = 2, 12, 2816
    assert splits(B, H, N)
    rng = np.random.default_rng(4400)
    valid = rng.random((B, N)) >= 0.1
    valid[1, 2100:] = False
    q, k, v = inputs(B, H, N, seed=4401)
    bits = ea.pack_key_mask(torch.from_numpy(valid).to(DEV))
    kl = torch.tensor([N, 2100], dtype=torch.int32, device=DEV)
    o, lse, _ = run_split(*(t.to(DEV) for t in (q, k, v)), key_len=kl, key_bits=bits)
    check(q, k, v, o, lse, "split with key mask", key_valid=valid)


def _random_split_cases(count=8, seed=5150):
    """Shapes drawn until the library splits them on 256 CUs (at most 200,000 rows, so
    the oracle stays fast), each with no mask, valid lengths or a random
    mask, at the workloads' scale or a sharper one."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        N, B, H = int(rng.integers(2048, 4200)), int(rng.integers(1, 3)), int(rng.integers(1, 80))
        mask = str(rng.choice(["none", "len", "valid"]))
        scale = float(0.125 if rng.random() < 0.6 else rng.uniform(-0.5, 1.0))
        seed_i = int(rng.integers(0, 2**31))
        if B * H * N <= 200_000 and splits_at(B, H, N, 256):  # drawn for a 256-CU MI355X
            cases.append(dict(B=B, H=H, N=N, mask=mask, scale=scale, seed=seed_i))
    return cases


@pytest.mark.parametrize("case", _random_split_cases(), ids=lambda c: "B%dH%dN%d_%s" % (c["B"], c["H"], c["N"], c["mask"]))
def test_random_split_calls(case):
    """forward() on random shapes, masks and scales; the cases the library
    splits are compared with the oracle on every row (the others run the
    plain kernel, covered elsewhere)."""
    B, H, N, scale = case["B"], case["H"], case["N"], case["scale"]
    if not splits(B, H, N):
        pytest.skip("not split on this part")
    print(f"[case] {case}", flush=True)
    q, k, v = make_inputs(Workload("split_fuzz", B, H, N, 64, "bf16", 1.0, scale, False, case["seed"], ""))
    rng = np.random.default_rng(case["seed"])
    kwargs, valid = {}, None
    if case["mask"] == "len":
        lens = rng.integers(0, N + 1, size=B)
        valid = np.arange(N)[None, :] < lens[:, None]
        kwargs = dict(key_len=torch.tensor(lens, dtype=torch.int32, device=DEV))
    elif case["mask"] == "valid":
        valid = rng.random((B, N)) < rng.uniform(0.3, 1.0)
        kwargs = dict(key_valid=torch.from_numpy(valid).to(DEV))
    o, lse = ea.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, **kwargs)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), scale, key_valid=valid)
    o_h, lse_h = to_f64(o), to_f64(lse)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_h), empty), "rows that see no key differ"
    assert np.all(o_h[empty] == 0.0)
    keep = ~empty
    if not keep.any():
        return
    if scale == 0.125:
        assert_within(errors(o_h[keep], lse_h[keep], o_ref[keep], lse_ref[keep]), BF16, str(case))
    else:
        o_abs, _ = oracle_attention(to_f64(q), to_f64(k), np.abs(to_f64(v)), scale, key_valid=valid)
        assert_bf16_elementwise(o_h[keep], lse_h[keep], o_ref[keep], lse_ref[keep], o_abs[keep], str(case))


def test_split_strided_views_match_contiguous_bitwise():
    """Head views of one packed [B, N, 3*H*d] projection: the same pieces as
    the contiguous call, hence the same bits."""
    B, H, N, d = 1, 24, 2816, 64
    assert splits(B, H, N)
    q, k, v = (t.to(DEV) for t in inputs(B, H, N, seed=4500))
    x = torch.empty(B, N, 3 * H * d, dtype=q.dtype, device=DEV)
    qs, ks, vs = (t.view(B, N, H, d).transpose(1, 2) for t in x.chunk(3, dim=-1))
    for dst, src in ((qs, q), (ks, k), (vs, v)):
        dst.copy_(src)
    o_c, l_c = ea.forward(q, k, v, scale=0.125)
    o_s, l_s = ea.forward(qs, ks, vs, scale=0.125)
    torch.cuda.synchronize()
    assert not qs.is_contiguous()
    assert torch.equal(o_s, o_c) and torch.equal(l_s, l_c)


def test_split_nan_rows_follow_the_definition():
    """A NaN in one K row makes every row NaN (all rows see every key); a NaN
    in feature 5 of one V row makes column 5 of O NaN and nothing else."""
    B, H, N = 1, 24, 2816
    assert splits(B, H, N)
    q, k, v = inputs(B, H, N, seed=4600)
    k[0, 0, 2000] = float("nan")
    v[0, 1, 1234, 5] = float("nan")
    o, lse, _ = run_split(*(t.to(DEV) for t in (q, k, v)))
    o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), 0.125)
    o_h, lse_h = to_f64(o), to_f64(lse)
    assert np.array_equal(np.isnan(o_h), np.isnan(o_ref)), "NaN positions of O"
    assert np.array_equal(np.isnan(lse_h), np.isnan(lse_ref)), "NaN positions of LSE"
    ok = ~np.isnan(o_ref)
    assert np.isnan(o_ref[0, 0]).all() and np.isnan(o_ref[0, 1, :, 5]).all() and ok[0, 2:].all()
    e = errors(np.where(ok, o_h, 0), np.where(np.isnan(lse_ref), 0, lse_h),
               np.where(ok, o_ref, 0), np.where(np.isnan(lse_ref), 0, lse_ref))
    assert_within(e, {kk: vv for kk, vv in BF16.items() if kk != "o_mean"}, "finite parts")


def test_split_infinite_inputs_follow_the_definition():
    """Head 2's last query tile is split (1 x 24 x 2816: one leftover tile
    per XCD).  K[2000, 5] = +inf there: rows with q[5] > 0 score +inf (NaN
    rows: some piece's reference max is +inf and the merge takes
    2^(inf - inf)), rows with q[5] < 0 score -inf (the key takes no part),
    rows with q[5] = 0 score NaN.  V[1234, 5] = -inf in head 5 (also split):
    column 5 of O is -inf in every row."""
    B, H, N, F = 1, 24, 2816, 5
    assert splits(B, H, N)
    q, k, v = inputs(B, H, N, seed=4650)
    k[0, 2, 2000, F] = float("inf")
    mag = q[0, 2, :, F].abs() + 0.25
    r = torch.arange(N)
    q[0, 2, :, F] = torch.where(r % 3 == 0, torch.zeros_like(mag), torch.where(r % 3 == 1, mag, -mag))
    v[0, 5, 1234, F] = float("-inf")
    o, lse, _ = run_split(*(t.to(DEV) for t in (q, k, v)))
    with np.errstate(invalid="ignore"):
        o_ref, lse_ref = oracle_attention(to_f64(q), to_f64(k), to_f64(v), 0.125)
    o_h, lse_h = to_f64(o), to_f64(lse)
    rr = np.arange(N)
    assert np.isnan(lse_ref[0, 2, rr % 3 != 2]).all() and np.isfinite(lse_ref[0, 2, rr % 3 == 2]).all()
    assert np.isneginf(o_ref[0, 5, :, F]).all()
    assert np.array_equal(np.isnan(o_h), np.isnan(o_ref)), "NaN positions of O"
    assert np.array_equal(np.isnan(lse_h), np.isnan(lse_ref)), "NaN positions of LSE"
    assert np.array_equal(np.isneginf(o_h), np.isneginf(o_ref)), "-inf positions of O"
    ok = np.isfinite(o_ref)
    e = errors(np.where(ok, o_h, 0), np.where(np.isnan(lse_ref), 0, lse_h),
               np.where(ok, o_ref, 0), np.where(np.isnan(lse_ref), 0, lse_ref))
    assert_within(e, {kk: vv for kk, vv in BF16.items() if kk != "o_mean"}, "finite parts")


def test_split_replays_in_a_graph():
    """forward() captured on a fresh stream (its workspace then comes from
    the graph's pool, the counter block cleared by a captured fill) and
    replayed with eager work between replays: every replay gives the eager
    bits."""
    B, H, N = SHAPES[2]
    q, k, v = (t.to(DEV) for t in inputs(B, H, N, seed=4700))
    o_ref, l_ref = ea.forward(q, k, v, scale=0.125)
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            for _ in range(3):  # several split calls per replay, each clearing its counters
                ea.forward(q, k, v, scale=0.125, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for replay in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        filler = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(filler)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"replay {replay} differs"


def test_split_graphs_and_eager_calls_keep_their_own_workspaces():
    """Two graphs captured back to back on one stream, an eager call on that
    stream before any replay, then the graphs replayed in the other order
    and at once on two streams: each captured call has a workspace of its
    own (cleared by its own captured fill), so none of these shares arrival
    counters or partial slots with another, and every result has the eager
    bits."""
    B, H, N = SHAPES[2]
    q, k, v = (t.to(DEV) for t in inputs(B, H, N, seed=4750))
    o_ref, l_ref = ea.forward(q, k, v, scale=0.125)
    torch.cuda.synchronize()
    outs = [(torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=DEV)) for _ in range(2)]
    graphs = [torch.cuda.CUDAGraph() for _ in range(2)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for g, (o, lse) in zip(graphs, outs):
            with torch.cuda.graph(g, stream=side):
                ea.forward(q, k, v, scale=0.125, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert (DEV_INDEX, side.cuda_stream) not in ea._SPLIT_WS  # captures keep no eager workspace
    with torch.cuda.stream(side):
        o_e, l_e = ea.forward(q, k, v, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o_e, o_ref) and torch.equal(l_e, l_ref), "eager call after the captures"
    for o, lse in outs:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    torch.cuda.synchronize()
    graphs[1].replay()
    torch.cuda.synchronize()
    graphs[0].replay()
    torch.cuda.synchronize()
    for i, (o, lse) in enumerate(outs):
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"graph {i}, replayed in reverse order"
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    for g, st in zip(graphs, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            g.replay()
    torch.cuda.synchronize()
    for i, (o, lse) in enumerate(outs):
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"graph {i}, replayed beside the other"


def test_split_workspace_validation():
    B, H, N = SHAPES[0]
    q, k, v = (t.to(DEV) for t in inputs(B, H, N, seed=4800))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    need = ea.attn_fwd_split_workspace_size(B, H, N, False)
    assert ea.attn_fwd_split_workspace_size(B, H, N, True) == 0      # causal: never split
    assert ea.attn_fwd_split_workspace_size(1, 16, 11616, False) == 0  # a 7/8-full last round: not split
    c = cus() // 8
    # the counters (8*C ints, padded to 256 bytes), then 2 slots of 69,632 bytes per range
    assert need == (8 * c * 4 + 255) // 256 * 256 + 16 * c * 69632
    ws = torch.zeros(need + 512, dtype=torch.uint8, device=DEV)
    lib = ea.load_library()
    stream = torch.cuda.current_stream().cuda_stream

    def call(ptr, size):
        return lib.attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, H, N, 64, 0.125, 0, None, None, None, None, None, None, ptr, size, stream)
    assert call(None, need) == ea.ATTN_E_INVALID
    assert call(ws.data_ptr() + 16, need) == ea.ATTN_E_ALIGN
    assert call(ws.data_ptr(), need - 1) == ea.ATTN_E_INVALID
    assert call(ws.data_ptr(), need) == ea.ATTN_OK
    torch.cuda.synchronize()
    assert int(ws[:count_bytes()].count_nonzero()) == 0


def test_unsplit_calls_take_no_workspace():
    """A call attn_fwd_split does not split runs with a NULL workspace and
    gives attn_fwd's bits; forward() then makes no workspace."""
    B, H, N = 1, 16, 2000
    assert not splits(B, H, N) and ea.attn_fwd_split_workspace_size(B, H, N, False) == 0
    q, k, v = (t.to(DEV) for t in inputs(B, H, N, seed=4900))
    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        assert ea.load_library().attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                                lse.data_ptr(), B, H, N, 64, 0.125, 0, None, None, None, None,
                                                None, None, None, 0, stream.cuda_stream) == ea.ATTN_OK
        o_f, l_f = ea.forward(q, k, v, scale=0.125)
    torch.cuda.synchronize()
    o0, l0 = ea.forward(q, k, v, scale=0.125, split=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0) and torch.equal(o_f, o0)
    assert (DEV_INDEX, stream.cuda_stream) not in ea._SPLIT_WS
