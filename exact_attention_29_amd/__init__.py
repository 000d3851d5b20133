"""Exact attention forward on MI355X: a thin Python binding over libattn.so.

The functions ``attn_fwd``, ``attn_fwd_fp32``, ``attn_fwd_masked``,
``attn_fwd_fp32_masked``, ``attn_fwd_strided``, ``attn_fwd_split``,
``attn_fwd_split_workspace_size``, ``attn_fwd_block_sparse``,
``attn_bwd``, ``attn_bwd_masked``, ``attn_bwd_strided``, ``attn_bwd_block_sparse``, ``attn_bwd_noalloc``,
``attn_bwd_workspace_size``,
``attn_pack_key_mask`` and ``attn_strerror`` carry the names and
arguments
of the C entry points declared in include/attn.h and only marshal arguments;
every step of the computation runs in the HIP kernels.
``forward`` is a convenience wrapper that allocates the outputs (and the
split workspace: once per device and stream, or per captured call) with
torch and launches on torch's current stream.  There is no CPU fallback:
without the built library (or without a gfx950 device) every call raises.
"""

import ctypes
import os

import torch  # imported first: the library then binds to torch's HIP runtime

__all__ = ["attn_fwd", "attn_fwd_fp32", "attn_fwd_masked", "attn_fwd_fp32_masked",
           "attn_fwd_strided", "attn_fwd_split", "attn_fwd_split_workspace_size", "attn_fwd_block_sparse", "attn_bwd", "attn_bwd_masked", "attn_bwd_strided", "attn_bwd_block_sparse",
           "attn_bwd_noalloc", "attn_bwd_workspace_size", "attn_pack_key_mask", "AttnLayout",
           "backward", "attn_strerror", "forward", "pack_key_mask", "AttnError",
           "library_path", "load_library", "split_workspace"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn.so")
_lib = None

ATTN_OK, ATTN_E_INVALID, ATTN_E_ALIGN, ATTN_E_DEVICE, ATTN_E_LAUNCH, ATTN_E_SCRATCH = range(6)
# the static scratch of attn_bwd_noalloc (ATTN_BWD_NOALLOC_SCRATCH_BYTES in attn.h)
BWD_NOALLOC_SCRATCH_BYTES = 16 << 20
EXPORTED = ("attn_bwd", "attn_bwd_masked", "attn_bwd_strided", "attn_bwd_block_sparse", "attn_bwd_noalloc", "attn_bwd_workspace_size", "attn_fwd", "attn_fwd_fp32", "attn_fwd_masked", "attn_fwd_fp32_masked",
            "attn_fwd_strided", "attn_fwd_split", "attn_fwd_split_workspace_size", "attn_fwd_block_sparse",
            "attn_pack_key_mask", "attn_strerror")
SPARSE_BLOCK_Q, SPARSE_BLOCK_K = 128, 64


class AttnLayout(ctypes.Structure):
    """attn_layout: element strides (batch, head, row) of a [B, H, N, d] tensor."""
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong), ("row", ctypes.c_longlong)]


class AttnError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{message} (status {code})")
        self.code = code


def library_path():
    return _LIB_PATH


def load_library():
    """Load libattn.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"HIP library not built: {_LIB_PATH} is missing "
            "(run `python exact_attention_29_amd/build.py` first)")
    lib = ctypes.CDLL(_LIB_PATH)
    ptr, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sig = [ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, f32, i32, ptr]
    lib.attn_fwd.argtypes = sig
    lib.attn_fwd.restype = i32
    lib.attn_fwd_fp32.argtypes = sig
    lib.attn_fwd_fp32.restype = i32
    msig = [ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, f32, i32, ptr, ptr, ptr]
    lib.attn_fwd_masked.argtypes = msig
    lib.attn_fwd_masked.restype = i32
    lib.attn_fwd_fp32_masked.argtypes = msig
    lib.attn_fwd_fp32_masked.restype = i32
    lay = ctypes.POINTER(AttnLayout)
    lib.attn_fwd_strided.argtypes = [ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, f32, i32,
                                     lay, lay, lay, lay, ptr, ptr, ptr]
    lib.attn_fwd_strided.restype = i32
    lib.attn_fwd_split.argtypes = [ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, f32, i32,
                                   lay, lay, lay, lay, ptr, ptr, ptr, ctypes.c_size_t, ptr]
    lib.attn_fwd_split.restype = i32
    lib.attn_fwd_split_workspace_size.argtypes = [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_fwd_split_workspace_size.restype = i32
    lib.attn_fwd_block_sparse.argtypes = [ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, f32, i32, ptr, ptr]
    lib.attn_fwd_block_sparse.restype = i32
    lib.attn_bwd.argtypes = [ptr] * 10 + [i32, i32, i32, i32, f32, i32, ptr]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_masked.argtypes = [ptr] * 10 + [i32, i32, i32, i32, f32, i32, ptr, ptr, ptr]
    lib.attn_bwd_masked.restype = i32
    lib.attn_bwd_strided.argtypes = [ptr] * 10 + [i32, i32, i32, i32, f32, i32] + [lay] * 8 + [ptr, ptr, ptr]
    lib.attn_bwd_strided.restype = i32
    lib.attn_bwd_block_sparse.argtypes = [ptr] * 10 + [i32, i32, i32, i32, f32, i32, ptr, ptr]
    lib.attn_bwd_block_sparse.restype = i32
    lib.attn_bwd_noalloc.argtypes = [ptr] * 9 + [i32, i32, i32, i32, f32, i32, ptr]
    lib.attn_bwd_noalloc.restype = i32
    lib.attn_bwd_workspace_size.argtypes = [i32, i32, i32]
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_pack_key_mask.argtypes = [ptr, ptr, i32, i32, ptr]
    lib.attn_pack_key_mask.restype = i32
    lib.attn_strerror.argtypes = [i32]
    lib.attn_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_strerror(status):
    return load_library().attn_strerror(int(status)).decode()


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, attn_strerror(status))


def attn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream):
    """C entry point attn_fwd: q, k, v, o, lse and stream are raw addresses (int)."""
    _check(load_library().attn_fwd(q, k, v, o, lse, B, H, N, d, float(scale), int(bool(causal)), stream))


def attn_fwd_fp32(q, k, v, o, lse, B, H, N, d, scale, causal, stream):
    """C entry point attn_fwd_fp32: raw addresses as in attn_fwd."""
    _check(load_library().attn_fwd_fp32(q, k, v, o, lse, B, H, N, d, float(scale), int(bool(causal)), stream))


def attn_fwd_masked(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, key_bits, stream):
    """C entry point attn_fwd_masked: raw addresses; key_len and key_bits may be 0 (NULL)."""
    _check(load_library().attn_fwd_masked(q, k, v, o, lse, B, H, N, d, float(scale), int(bool(causal)),
                                          key_len, key_bits, stream))


def attn_fwd_fp32_masked(q, k, v, o, lse, B, H, N, d, scale, causal, key_len, key_bits, stream):
    """C entry point attn_fwd_fp32_masked: raw addresses as in attn_fwd_masked."""
    _check(load_library().attn_fwd_fp32_masked(q, k, v, o, lse, B, H, N, d, float(scale), int(bool(causal)),
                                               key_len, key_bits, stream))


def attn_fwd_strided(q, k, v, o, lse, B, H, N, d, scale, causal, q_layout, k_layout, v_layout,
                     o_layout, key_len, key_bits, stream):
    """C entry point attn_fwd_strided: raw addresses; layouts are AttnLayout or None (contiguous)."""
    ref = lambda l: None if l is None else ctypes.byref(l)  # noqa: E731
    _check(load_library().attn_fwd_strided(q, k, v, o, lse, B, H, N, d, float(scale), int(bool(causal)),
                                           ref(q_layout), ref(k_layout), ref(v_layout), ref(o_layout),
                                           key_len, key_bits, stream))


def attn_fwd_split(q, k, v, o, lse, B, H, N, d, scale, causal, q_layout, k_layout, v_layout,
                   o_layout, key_len, key_bits, workspace, workspace_bytes, stream):
    """C entry point attn_fwd_split: attn_fwd_strided plus a workspace (raw
    address and size in bytes; layouts AttnLayout or None)."""
    _check(load_library().attn_fwd_split(q, k, v, o, lse, B, H, N, d, float(scale), int(bool(causal)),
                                         q_layout, k_layout, v_layout, o_layout, key_len, key_bits,
                                         workspace, workspace_bytes, stream))


def attn_fwd_split_workspace_size(B, H, N, causal):
    """C entry point attn_fwd_split_workspace_size: bytes of workspace the
    call needs on the current device (0: not split)."""
    n = ctypes.c_size_t(0)
    _check(load_library().attn_fwd_split_workspace_size(B, H, N, int(bool(causal)), ctypes.byref(n)))
    return n.value


def attn_fwd_block_sparse(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, stream):
    """C entry point attn_fwd_block_sparse: raw addresses; block_mask [ceil(N/128)][ceil(N/64)] bytes."""
    _check(load_library().attn_fwd_block_sparse(q, k, v, o, lse, B, H, N, d, float(scale), int(bool(causal)),
                                                block_mask, stream))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale, causal, stream):
    """C entry point attn_bwd: raw addresses of the nine tensors and the workspace."""
    _check(load_library().attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, float(scale),
                                   int(bool(causal)), stream))


def attn_bwd_masked(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale, causal, key_len, key_bits,
                    stream):
    """C entry point attn_bwd_masked: attn_bwd plus the device addresses of
    the int32 [B] valid key lengths and the [B, ceil(N/32)] key bit words
    (0 = none)."""
    _check(load_library().attn_bwd_masked(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, float(scale),
                                          int(bool(causal)), key_len, key_bits, stream))


def attn_bwd_strided(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale, causal, layouts, key_len,
                     key_bits, stream):
    """C entry point attn_bwd_strided: attn_bwd_masked plus the layouts of q,
    k, v, o, dout, dq, dk, dv (a sequence of eight AttnLayout or None)."""
    ref = lambda l: None if l is None else ctypes.byref(l)  # noqa: E731
    _check(load_library().attn_bwd_strided(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, float(scale),
                                           int(bool(causal)), *[ref(l) for l in layouts], key_len, key_bits,
                                           stream))


def attn_bwd_block_sparse(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale, causal, block_mask,
                          stream):
    """C entry point attn_bwd_block_sparse: attn_bwd plus the device address
    of the [ceil(N/128)][ceil(N/64)] block mask bytes."""
    _check(load_library().attn_bwd_block_sparse(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d,
                                                float(scale), int(bool(causal)), block_mask, stream))


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, stream):
    """C entry point attn_bwd_noalloc: attn_bwd without a workspace argument
    (the library's static device scratch; allocates nothing)."""
    _check(load_library().attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, float(scale),
                                           int(bool(causal)), stream))


def attn_bwd_workspace_size(B, H, N):
    """C entry point attn_bwd_workspace_size: bytes of workspace attn_bwd needs."""
    return int(load_library().attn_bwd_workspace_size(B, H, N))


def backward(q, k, v, o, lse, dout, scale=None, causal=False, key_len=None, key_valid=None, key_bits=None,
             block_mask=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV (bf16 [B, H, N, d]) of attention for upstream gradient dout,
    from forward's o and lse (same q, k, v, scale, causal and masks).
    Key masks as in forward (int32 [B] key_len, bool [B, N] key_valid packed
    here, or int32 [B, ceil(N/32)] key_bits), through attn_bwd_masked:
    hidden keys get dK = dV = 0.  block_mask as in forward (bool or uint8
    [ceil(N/128), ceil(N/64)], no key mask), through attn_bwd_block_sparse.
    bf16 tensors on one GPU; q, k, v, o, dout may be strided views (features
    contiguous, every stride a multiple of 8 elements), and dq, dk, dv may be
    given as such views to write into (e.g. head views of a packed
    projection's gradient); then attn_bwd_strided runs (no block mask).
    The workspace (attn_bwd_workspace_size bytes) is allocated here.
    Launches on torch's current stream."""
    ts = (q, k, v, o, dout)
    if any(t.dtype != torch.bfloat16 or t.shape != q.shape or t.device != q.device for t in ts) \
            or q.dim() != 4 or not q.is_cuda:
        raise ValueError("q, k, v, o, dout must be bf16 [B, H, N, d] tensors on one GPU")
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    dq, dk, dv = (torch.empty_like(q, memory_format=torch.contiguous_format) if g is None else g
                  for g in (dq, dk, dv))
    if any(g.dtype != torch.bfloat16 or g.shape != q.shape or g.device != q.device for g in (dq, dk, dv)):
        raise ValueError("dq, dk, dv must be bf16 [B, H, N, d] tensors like q")
    strided = not all(t.is_contiguous() for t in (*ts, dq, dk, dv))
    if B * H * N == 0 and d == 64:
        return dq, dk, dv  # nothing to compute (the C entry points take B, H, N >= 1)
    if key_len is not None and (key_len.dtype != torch.int32 or key_len.shape != (B,)
                                or not key_len.is_contiguous() or key_len.device != q.device):
        raise ValueError("key_len must be a contiguous int32 [B] tensor on q's device")
    if key_valid is not None:
        if key_bits is not None:
            raise ValueError("give key_valid or key_bits, not both")
        if key_valid.shape != (B, N) or key_valid.device != q.device:
            raise ValueError("key_valid must be a [B, N] tensor on q's device")
        key_bits = pack_key_mask(key_valid)
    if key_bits is not None and (key_bits.dtype != torch.int32 or key_bits.shape != (B, (N + 31) // 32)
                                 or not key_bits.is_contiguous() or key_bits.device != q.device):
        raise ValueError("key_bits must be a contiguous int32 [B, ceil(N/32)] tensor on q's device")
    if block_mask is not None:
        nbq, nbk = (N + 127) // 128, (N + 63) // 64
        if block_mask.dtype not in (torch.bool, torch.uint8) or block_mask.shape != (nbq, nbk) \
                or not block_mask.is_contiguous() or block_mask.device != q.device:
            raise ValueError(f"block_mask must be a contiguous bool or uint8 [{nbq}, {nbk}] tensor on q's device")
        if key_len is not None or key_bits is not None or strided:
            raise ValueError("block_mask takes contiguous tensors and no key mask")
    ws = torch.empty(attn_bwd_workspace_size(B, H, N), dtype=torch.uint8, device=q.device)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr())
    with torch.cuda.device(q.device):
        if block_mask is not None:
            attn_bwd_block_sparse(*ptrs, B, H, N, d, scale, causal, block_mask.data_ptr(), _stream_handle(q.device))
        elif strided:
            attn_bwd_strided(*ptrs, B, H, N, d, scale, causal, [_layout(t) for t in (*ts, dq, dk, dv)],
                             0 if key_len is None else key_len.data_ptr(),
                             0 if key_bits is None else key_bits.data_ptr(), _stream_handle(q.device))
        elif key_len is None and key_bits is None:
            attn_bwd(*ptrs, B, H, N, d, scale, causal, _stream_handle(q.device))
        else:
            attn_bwd_masked(*ptrs, B, H, N, d, scale, causal, 0 if key_len is None else key_len.data_ptr(),
                            0 if key_bits is None else key_bits.data_ptr(), _stream_handle(q.device))
    return dq, dk, dv


def attn_pack_key_mask(key_valid, key_bits, B, N, stream):
    """C entry point attn_pack_key_mask: raw addresses of the byte mask and the bit words."""
    _check(load_library().attn_pack_key_mask(key_valid, key_bits, B, N, stream))


def pack_key_mask(key_valid):
    """Bit words [B, ceil(N/32)] (int32) of a bool or uint8 [B, N] device mask,
    built by attn_pack_key_mask on torch's current stream."""
    if key_valid.dtype not in (torch.bool, torch.uint8) or key_valid.dim() != 2 \
            or not key_valid.is_contiguous() or not key_valid.is_cuda:
        raise ValueError("key_valid must be a contiguous bool or uint8 [B, N] GPU tensor")
    B, N = key_valid.shape
    bits = torch.empty((B, (N + 31) // 32), dtype=torch.int32, device=key_valid.device)
    with torch.cuda.device(key_valid.device):
        attn_pack_key_mask(key_valid.data_ptr(), bits.data_ptr(), B, N, _stream_handle(key_valid.device))
    return bits


def _stream_handle(device):
    return torch.cuda.current_stream(device).cuda_stream


# forward()'s split workspaces for eager calls: one per (device index,
# stream handle), so that calls on different streams never share one
_SPLIT_WS = {}
# the first bytes of a workspace hold the arrival counters (at most 64 ints
# per XCD, 8 XCDs); attn_fwd_split needs them zero at the start of a call
_SPLIT_COUNT_BYTES = 2048


def split_workspace(device, stream, n):
    """The workspace forward() hands attn_fwd_split on (device, stream): a
    uint8 tensor of n bytes (what attn_fwd_split_workspace_size reports for
    a split call; the same for every split call on a device) whose counters
    are zero when the call starts.

    Eager calls share one per stream, made zeroed on first use; every
    completed call leaves its counters zero again.  A call under graph
    capture gets one of its own from the graph's memory pool, its counter
    block cleared by a fill kernel captured just before the call, so every
    replay starts from zero whatever ran before it, and a replay (on
    whatever stream) shares no workspace with eager calls or other graphs.
    It is released when forward() returns; the pool can hand the same
    block to the capture's next split call on that stream, which runs after
    this one in every replay."""
    if torch.cuda.is_current_stream_capturing():
        ws = torch.empty(n, dtype=torch.uint8, device=device)
        ws[:_SPLIT_COUNT_BYTES].zero_()
        return ws
    key = (device.index, stream)
    ws = _SPLIT_WS.get(key)
    if ws is None or ws.numel() < n:
        ws = torch.zeros(n, dtype=torch.uint8, device=device)
        _SPLIT_WS[key] = ws
    return ws


def _layout(t):
    """AttnLayout of a [B, H, N, d] tensor view with contiguous features."""
    sb, sh, sn, sf = t.stride()
    if sf != 1:
        raise ValueError("the d features of every tensor must be contiguous (stride 1)")
    return AttnLayout(sb, sh, sn)


def forward(q, k, v, scale=None, causal=False, out=None, lse=None, key_len=None, key_valid=None,
            key_bits=None, block_mask=None, split=True):
    """O, LSE for [B, H, N, d] tensors on one device.

    bf16 tensors use attn_fwd, fp32 tensors attn_fwd_fp32.  ``scale``
    defaults to 1/sqrt(d).  ``out`` and ``lse`` may be given to reuse buffers.
    bf16 q, k, v and out may be strided views (features contiguous, every
    stride a multiple of 8 elements), e.g. head views of one packed input
    projection; then attn_fwd_strided reads them in place.
    Key padding: ``key_len`` an int32 [B] tensor (keys j >= key_len[b] take no
    part) and/or ``key_valid`` a bool or uint8 [B, N] tensor (key j of entry b
    takes part where it is True / non-zero; packed to bits by
    attn_pack_key_mask first) or ``key_bits`` the packed int32
    [B, ceil(N/32)] words, all on the same device; then the masked entry
    points are called.  Rows that see no key get O = 0 and LSE = -inf.
    Block-sparse: ``block_mask`` a bool or uint8 [ceil(N/128), ceil(N/64)]
    tensor on the same device (query blocks of 128 rows, key blocks of 64
    keys; only set blocks are computed), with contiguous bf16 q, k, v, out
    and no key mask (attn_fwd_block_sparse).
    Non-causal bf16 calls without a block mask that attn_fwd_split would
    split (a mostly empty last round of workgroups; unless ``split=False``)
    go through it, with the workspace split_workspace() keeps for the device
    and stream (under graph capture, one of the graph's own).
    Launches on torch's current stream and returns without synchronising.
    """
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share one dtype")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"unsupported dtype {q.dtype}; use bfloat16 or float32")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one 4-D shape [B, H, N, d]")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must live on one GPU")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if out is None:
        out = torch.empty((B, H, N, d), dtype=q.dtype, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device:
        raise ValueError("out must be a [B, H, N, d] tensor like q")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if B * H * N == 0 and d == 64:
        return out, lse  # nothing to compute (the C entry points take B, H, N >= 1)
    strided = not all(t.is_contiguous() for t in (q, k, v, out))
    if block_mask is not None:
        nbq, nbk = -(-N // SPARSE_BLOCK_Q), -(-N // SPARSE_BLOCK_K)
        if block_mask.dtype not in (torch.bool, torch.uint8) or block_mask.shape != (nbq, nbk) \
                or not block_mask.is_contiguous() or block_mask.device != q.device:
            raise ValueError(f"block_mask must be a contiguous bool or uint8 [{nbq}, {nbk}] tensor on q's device")
        if strided or q.dtype != torch.bfloat16 or key_len is not None or key_valid is not None \
                or key_bits is not None:
            raise ValueError("block_mask takes contiguous bf16 tensors and no key mask")
        with torch.cuda.device(q.device):
            attn_fwd_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  B, H, N, d, scale, causal, block_mask.data_ptr(), _stream_handle(q.device))
        return out, lse
    if strided and q.dtype != torch.bfloat16:
        raise ValueError("fp32 q, k, v and out must be contiguous [B, H, N, d]")
    if key_valid is not None:
        if key_bits is not None:
            raise ValueError("give key_valid or key_bits, not both")
        if key_valid.shape != (B, N) or key_valid.device != q.device:
            raise ValueError("key_valid must be a [B, N] tensor on q's device")
        key_bits = pack_key_mask(key_valid)
    kl_ptr = kv_ptr = 0
    if key_len is not None:
        if key_len.dtype != torch.int32 or key_len.shape != (B,) or not key_len.is_contiguous() \
                or key_len.device != q.device:
            raise ValueError("key_len must be a contiguous int32 [B] tensor on q's device")
        kl_ptr = key_len.data_ptr()
    if key_bits is not None:
        if key_bits.dtype != torch.int32 or key_bits.shape != (B, (N + 31) // 32) \
                or not key_bits.is_contiguous() or key_bits.device != q.device:
            raise ValueError("key_bits must be a contiguous int32 [B, ceil(N/32)] tensor on q's device")
        kv_ptr = key_bits.data_ptr()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    with torch.cuda.device(q.device):
        stream = _stream_handle(q.device)
        need = attn_fwd_split_workspace_size(B, H, N, causal) if split and not causal \
            and q.dtype == torch.bfloat16 else 0
        if need:
            ws = split_workspace(q.device, stream, need)
            lays = [_layout(t) if strided else None for t in (q, k, v, out)]
            attn_fwd_split(*ptrs, B, H, N, d, scale, causal, *lays, kl_ptr, kv_ptr, ws.data_ptr(), ws.numel(),
                           stream)
        elif strided:
            attn_fwd_strided(*ptrs, B, H, N, d, scale, causal, _layout(q), _layout(k), _layout(v),
                             _layout(out), kl_ptr, kv_ptr, stream)
        elif kl_ptr or kv_ptr:
            fn = attn_fwd_masked if q.dtype == torch.bfloat16 else attn_fwd_fp32_masked
            fn(*ptrs, B, H, N, d, scale, causal, kl_ptr, kv_ptr, stream)
        else:
            fn = attn_fwd if q.dtype == torch.bfloat16 else attn_fwd_fp32
            fn(*ptrs, B, H, N, d, scale, causal, stream)
    return out, lse
