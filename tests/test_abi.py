"""The C-ABI library: it loads, exports every declared entry point, and its
host-side validation works without a GPU (no compute call is made here)."""

import ctypes
import os
import re

import pytest

import exact_attention_29_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(ea.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ea.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_library_exports_nothing_else_c_visible():
    # the only extern "C" symbols are the declared ones
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", ea.library_path()],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if " T " in line}
    attn = sorted(n for n in names if n.startswith("attn_"))
    assert attn == declared_functions()


def test_strerror_covers_every_status():
    texts = [ea.attn_strerror(s) for s in range(6)]
    assert texts[0] == "success"
    assert len(set(texts)) == 6
    assert ea.attn_strerror(99) == "unknown status"


ALIGNED = 0x100000  # a fake, 16-byte aligned address; never dereferenced


MASKED = ("attn_fwd_masked", "attn_fwd_fp32_masked")


def call(fn, **kw):
    args = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, o=ALIGNED, lse=ALIGNED,
                B=1, H=1, N=8, d=64, scale=0.125, causal=0, key_len=None, key_bits=None,
                stream=None)
    args.update(kw)
    lib = ea.load_library()
    head = (args["q"], args["k"], args["v"], args["o"], args["lse"],
            args["B"], args["H"], args["N"], args["d"], args["scale"], args["causal"])
    if fn in MASKED:
        return getattr(lib, fn)(*head, args["key_len"], args["key_bits"], args["stream"])
    return getattr(lib, fn)(*head, args["stream"])


ALL_FWD = ["attn_fwd", "attn_fwd_fp32", *MASKED]
# attn_fwd_strided shares attn_fwd_masked's validation path; its own checks are below


@pytest.mark.parametrize("fn", MASKED)
def test_masked_validation(fn):
    # misaligned key_len or key_bits are refused before any device check
    assert call(fn, key_len=ALIGNED + 2) == ea.ATTN_E_ALIGN
    assert call(fn, key_bits=ALIGNED + 1) == ea.ATTN_E_ALIGN
    assert call(fn, q=None, key_len=ALIGNED) == ea.ATTN_E_INVALID
    assert call(fn, N=0, key_bits=ALIGNED) == ea.ATTN_E_INVALID


def test_strided_validation():
    lib = ea.load_library()

    def strided(q_layout=None, k_layout=None, v_layout=None, o_layout=None, N=8, key_len=None):
        lay = lambda t: None if t is None else ctypes.byref(ea.AttnLayout(*t))  # noqa: E731
        return lib.attn_fwd_strided(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 2, N, 64, 0.125, 0,
                                    lay(q_layout), lay(k_layout), lay(v_layout), lay(o_layout),
                                    key_len, None, None)
    assert strided(q_layout=(0, 64, -64)) == ea.ATTN_E_INVALID        # negative stride
    assert strided(k_layout=(4096, 64, 196)) == ea.ATTN_E_ALIGN       # row not 16-byte multiple
    assert strided(v_layout=(4096, 12, 192)) == ea.ATTN_E_ALIGN       # head not 16-byte multiple
    assert strided(o_layout=(4096, 8, 56)) == ea.ATTN_E_INVALID       # o rows would overlap
    assert strided(k_layout=(0, 0, 1 << 23), N=200) == ea.ATTN_E_INVALID  # K offsets >= 2^31
    assert strided(key_len=ALIGNED + 2) == ea.ATTN_E_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert strided() == ea.ATTN_E_DEVICE
        assert strided(q_layout=(8192, 64, 128), k_layout=(0, 0, 64), o_layout=(8192, 64, 128)) \
            == ea.ATTN_E_DEVICE


def test_block_sparse_validation():
    lib = ea.load_library()
    f = lambda **kw: lib.attn_fwd_block_sparse(kw.get("q", ALIGNED), ALIGNED, ALIGNED, ALIGNED, ALIGNED,  # noqa: E731
                                                1, 1, kw.get("N", 300), 64, 0.125, 0,
                                                kw.get("m", ALIGNED + 3), None)
    assert f(m=None) == ea.ATTN_E_INVALID
    assert f(q=None) == ea.ATTN_E_INVALID
    assert f(N=64 * 4096 + 1) == ea.ATTN_E_INVALID
    assert f(q=ALIGNED + 2) == ea.ATTN_E_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert f() == ea.ATTN_E_DEVICE


def test_backward_validation():
    lib = ea.load_library()

    def bwd(**kw):
        ptrs = [kw.get(n, ALIGNED) for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "ws")]
        return lib.attn_bwd(*ptrs, kw.get("B", 1), 1, kw.get("N", 100), kw.get("d", 64), 0.125, 0, None)
    assert bwd(ws=None) == ea.ATTN_E_INVALID
    assert bwd(dq=None) == ea.ATTN_E_INVALID
    assert bwd(d=32) == ea.ATTN_E_INVALID
    assert bwd(N=0) == ea.ATTN_E_INVALID
    assert bwd(N=1 << 24) == ea.ATTN_E_INVALID
    assert bwd(B=1 << 26, N=1024) == ea.ATTN_E_INVALID
    assert bwd(dout=ALIGNED + 8) == ea.ATTN_E_ALIGN
    assert bwd(ws=ALIGNED + 4) == ea.ATTN_E_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert bwd(lse=ALIGNED + 4) == ea.ATTN_E_DEVICE
        assert bwd(B=1 << 20, N=64) == ea.ATTN_E_DEVICE   # 2^32 elements per tensor


def test_backward_masked_validation():
    """attn_bwd_masked: attn_bwd's checks plus 4-byte aligned key_len and
    key_bits (NULL allowed: both NULL is attn_bwd), all before any device
    call."""
    lib = ea.load_library()

    def bwd(**kw):
        ptrs = [kw.get(n, ALIGNED) for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "ws")]
        return lib.attn_bwd_masked(*ptrs, kw.get("B", 1), 1, kw.get("N", 100), kw.get("d", 64), 0.125, 0,
                                   kw.get("key_len", ALIGNED), kw.get("key_bits", ALIGNED), None)
    assert bwd(ws=None) == ea.ATTN_E_INVALID
    assert bwd(dk=None) == ea.ATTN_E_INVALID
    assert bwd(d=32) == ea.ATTN_E_INVALID
    assert bwd(N=1 << 24) == ea.ATTN_E_INVALID
    assert bwd(key_len=ALIGNED + 2) == ea.ATTN_E_ALIGN
    assert bwd(key_bits=ALIGNED + 2) == ea.ATTN_E_ALIGN
    assert bwd(ws=ALIGNED + 4) == ea.ATTN_E_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert bwd() == ea.ATTN_E_DEVICE
        assert bwd(key_len=None) == ea.ATTN_E_DEVICE
        assert bwd(key_len=None, key_bits=None) == ea.ATTN_E_DEVICE


def test_backward_strided_validation():
    """attn_bwd_strided: attn_bwd_masked's checks plus the eight layouts
    (strides non-negative multiples of 8 elements, outputs' rows at least 64
    apart, the tile loads' byte offsets below 2^31), all before any device
    call."""
    lib = ea.load_library()
    names = ("q", "k", "v", "o", "dout", "dq", "dk", "dv")

    def bwd(N=100, key_len=None, **lays):
        ptrs = [ALIGNED] * 10
        lay = [None if lays.get(n) is None else ctypes.byref(ea.AttnLayout(*lays[n])) for n in names]
        return lib.attn_bwd_strided(*ptrs, 1, 2, N, 64, 0.125, 0, *lay, key_len, None, None)
    assert bwd(q=(0, 64, -64)) == ea.ATTN_E_INVALID          # negative stride
    assert bwd(dout=(4096, 64, 196)) == ea.ATTN_E_ALIGN      # row not a 16-byte multiple
    assert bwd(v=(4096, 12, 192)) == ea.ATTN_E_ALIGN         # head not a 16-byte multiple
    assert bwd(dk=(4096, 8, 56)) == ea.ATTN_E_INVALID        # dK rows would overlap
    assert bwd(dq=(4096, 8, 0)) == ea.ATTN_E_INVALID
    assert bwd(k=(0, 0, 1 << 23), N=200) == ea.ATTN_E_INVALID     # K tile offsets >= 2^31
    assert bwd(dout=(0, 0, 1 << 23), N=200) == ea.ATTN_E_INVALID  # dO tile offsets >= 2^31
    assert bwd(o=(0, 0, 1 << 23), N=200) != ea.ATTN_E_INVALID     # O is read row by row
    assert bwd(q=(0, 0, 1 << 25)) == ea.ATTN_E_INVALID       # row stride above 2^24
    assert bwd(key_len=ALIGNED + 2) == ea.ATTN_E_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert bwd() == ea.ATTN_E_DEVICE
        assert bwd(q=(8192 * 3, 192, 3 * 128), k=(0, 0, 64), dk=(8192, 64, 128)) == ea.ATTN_E_DEVICE


def test_backward_block_sparse_validation():
    """attn_bwd_block_sparse: attn_bwd's checks, a block mask, N <= 262,144,
    all before any device call."""
    lib = ea.load_library()

    def bwd(**kw):
        ptrs = [kw.get(n, ALIGNED) for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "ws")]
        return lib.attn_bwd_block_sparse(*ptrs, kw.get("B", 1), 1, kw.get("N", 100), kw.get("d", 64), 0.125, 0,
                                         kw.get("mask", ALIGNED), None)
    assert bwd(mask=None) == ea.ATTN_E_INVALID
    assert bwd(ws=None) == ea.ATTN_E_INVALID
    assert bwd(d=32) == ea.ATTN_E_INVALID
    assert bwd(N=64 * 4096 + 1) == ea.ATTN_E_INVALID
    assert bwd(q=ALIGNED + 2) == ea.ATTN_E_ALIGN
    assert bwd(ws=ALIGNED + 4) == ea.ATTN_E_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert bwd() == ea.ATTN_E_DEVICE
        assert bwd(N=64 * 4096) == ea.ATTN_E_DEVICE


def test_backward_noalloc_validation():
    """attn_bwd_noalloc: attn_bwd's checks, then the static scratch limit
    (16 MiB = 8 * B * H * ceil(N/256) * 256 bytes), all before any device
    call."""
    lib = ea.load_library()

    def bwd(**kw):
        ptrs = [kw.get(n, ALIGNED) for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv")]
        return lib.attn_bwd_noalloc(*ptrs, kw.get("B", 1), kw.get("H", 1), kw.get("N", 100), kw.get("d", 64),
                                    0.125, 0, None)
    assert bwd(dq=None) == ea.ATTN_E_INVALID
    assert bwd(d=32) == ea.ATTN_E_INVALID
    assert bwd(N=0) == ea.ATTN_E_INVALID
    assert bwd(dout=ALIGNED + 8) == ea.ATTN_E_ALIGN
    # 16 heads: N = 131,072 fits exactly, one more row does not
    assert ea.attn_bwd_workspace_size(1, 16, 131072) == ea.BWD_NOALLOC_SCRATCH_BYTES
    assert bwd(H=16, N=131073) == ea.ATTN_E_SCRATCH
    assert bwd(B=8193, H=1, N=256) == ea.ATTN_E_SCRATCH
    assert "scratch" in ea.attn_strerror(ea.ATTN_E_SCRATCH)
    import torch
    if not torch.cuda.is_available():
        assert bwd(H=16, N=131072) == ea.ATTN_E_DEVICE
        assert bwd(B=8192, H=1, N=256) == ea.ATTN_E_DEVICE


def test_backward_workspace_size():
    # two fp32 values per row of every head, rows padded to a multiple of 256
    size = ea.attn_bwd_workspace_size
    assert size(1, 1, 1) == 2 * 256 * 4
    assert size(1, 1, 256) == 2 * 256 * 4
    assert size(1, 1, 257) == 2 * 512 * 4
    assert size(8, 12, 1024) == 2 * 8 * 12 * 1024 * 4
    assert size(1, 16, 11616) == 2 * 16 * 11776 * 4
    assert size(0, 1, 1) == 0 and size(1, 0, 1) == 0 and size(1, 1, 0) == 0


def test_pack_key_mask_validation():
    lib = ea.load_library()
    assert lib.attn_pack_key_mask(None, ALIGNED, 1, 8, None) == ea.ATTN_E_INVALID
    assert lib.attn_pack_key_mask(ALIGNED, None, 1, 8, None) == ea.ATTN_E_INVALID
    assert lib.attn_pack_key_mask(ALIGNED, ALIGNED, 0, 8, None) == ea.ATTN_E_INVALID
    assert lib.attn_pack_key_mask(ALIGNED, ALIGNED, 1, 0, None) == ea.ATTN_E_INVALID
    assert lib.attn_pack_key_mask(ALIGNED, ALIGNED, 1 << 30, 64, None) == ea.ATTN_E_INVALID
    assert lib.attn_pack_key_mask(ALIGNED, ALIGNED, 1, 1 << 24, None) == ea.ATTN_E_INVALID
    assert lib.attn_pack_key_mask(ALIGNED + 1, ALIGNED + 2, 1, 8, None) == ea.ATTN_E_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert lib.attn_pack_key_mask(ALIGNED + 1, ALIGNED, 2, 33, None) == ea.ATTN_E_DEVICE
        assert lib.attn_pack_key_mask(ALIGNED, ALIGNED, 1 << 16, 1 << 15, None) == ea.ATTN_E_DEVICE


@pytest.mark.parametrize("fn", ALL_FWD)
@pytest.mark.parametrize("bad, status", [
    (dict(q=None), ea.ATTN_E_INVALID),
    (dict(lse=None), ea.ATTN_E_INVALID),
    (dict(B=0), ea.ATTN_E_INVALID),
    (dict(H=-1), ea.ATTN_E_INVALID),
    (dict(N=0), ea.ATTN_E_INVALID),
    (dict(d=128), ea.ATTN_E_INVALID),
    (dict(d=32), ea.ATTN_E_INVALID),
    (dict(scale=float("nan")), ea.ATTN_E_INVALID),
    (dict(scale=float("inf")), ea.ATTN_E_INVALID),
    (dict(B=1 << 16, H=1 << 15, N=2), ea.ATTN_E_INVALID),   # 2^31 workgroup-sized row blocks
    (dict(B=1 << 8, H=1 << 8, N=1 << 20), ea.ATTN_E_INVALID),  # B*H*ceil(N/32) = 2^31
    (dict(N=1 << 24), ea.ATTN_E_INVALID),                   # a head's rows past 32-bit byte offsets
    (dict(q=ALIGNED + 8), ea.ATTN_E_ALIGN),
    (dict(v=ALIGNED + 2), ea.ATTN_E_ALIGN),
    (dict(o=ALIGNED + 4), ea.ATTN_E_ALIGN),
    (dict(lse=ALIGNED + 2), ea.ATTN_E_ALIGN),
])
def test_validation_rejects(fn, bad, status):
    assert call(fn, **bad) == status


@pytest.mark.parametrize("fn", ALL_FWD)
def test_valid_arguments_without_a_gpu_report_no_device(fn):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call(fn) == ea.ATTN_E_DEVICE
    assert call(fn, lse=ALIGNED + 4, causal=1, scale=-0.5, N=1) == ea.ATTN_E_DEVICE
    # tensors past 2^31 elements pass validation (64-bit offsets between heads)
    assert call(fn, B=1 << 12, H=1 << 12, N=2) == ea.ATTN_E_DEVICE
    assert call(fn, B=2, H=8200, N=2048) == ea.ATTN_E_DEVICE
    assert call(fn, N=(1 << 24) - 1) == ea.ATTN_E_DEVICE
    if fn in MASKED:
        assert call(fn, key_len=ALIGNED + 4, key_bits=ALIGNED + 8) == ea.ATTN_E_DEVICE


def test_binding_raises_without_compute_on_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.forward(q, q, q)
    with pytest.raises(TypeError):
        ea.forward(q.half(), q.half(), q.half())


def test_split_validation():
    lib = ea.load_library()

    def split(ws=ALIGNED, size=1 << 30, q=ALIGNED, N=8):
        return lib.attn_fwd_split(q, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 2, N, 64, 0.125, 0,
                                  None, None, None, None, None, None, ws, size, None)
    assert split(ws=ALIGNED + 16) == ea.ATTN_E_ALIGN     # 256-byte alignment, checked first
    assert split(q=None) == ea.ATTN_E_INVALID
    assert split(N=0) == ea.ATTN_E_INVALID
    assert split(q=ALIGNED + 2) == ea.ATTN_E_ALIGN
    n = ctypes.c_size_t(7)
    assert lib.attn_fwd_split_workspace_size(1, 1, 8, 0, None) == ea.ATTN_E_INVALID
    assert lib.attn_fwd_split_workspace_size(0, 1, 8, 0, ctypes.byref(n)) == ea.ATTN_E_INVALID
    assert lib.attn_fwd_split_workspace_size(1, 1, 1 << 24, 0, ctypes.byref(n)) == ea.ATTN_E_INVALID
    import torch
    if not torch.cuda.is_available():
        assert split() == ea.ATTN_E_DEVICE
        assert split(ws=None) == ea.ATTN_E_DEVICE
        assert lib.attn_fwd_split_workspace_size(1, 16, 38400, 0, ctypes.byref(n)) == ea.ATTN_E_DEVICE
    assert n.value == 7  # untouched on error
