"""Exact attention forward on MI355X: a thin Python binding over libattn.so.

The functions ``attn_fwd``, ``attn_fwd_fp32`` and ``attn_strerror`` carry the
names and arguments of the C entry points declared in include/attn.h and only
marshal arguments; every step of the computation runs in the HIP kernels.
``forward`` is a convenience wrapper that allocates the outputs with torch
and launches on torch's current stream.  There is no CPU fallback: without
the built library (or without a gfx950 device) every call raises.
"""

import ctypes
import os

import torch  # imported first: the library then binds to torch's HIP runtime

__all__ = ["attn_fwd", "attn_fwd_fp32", "attn_strerror", "forward", "AttnError",
           "library_path", "load_library"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn.so")
_lib = None

ATTN_OK, ATTN_E_INVALID, ATTN_E_ALIGN, ATTN_E_DEVICE, ATTN_E_LAUNCH = range(5)
EXPORTED = ("attn_fwd", "attn_fwd_fp32", "attn_strerror")


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
            "(run `python -c 'import __graft_entry__ as g; g.build()'` first)")
    lib = ctypes.CDLL(_LIB_PATH)
    ptr, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sig = [ptr, ptr, ptr, ptr, ptr, i32, i32, i32, i32, f32, i32, ptr]
    lib.attn_fwd.argtypes = sig
    lib.attn_fwd.restype = i32
    lib.attn_fwd_fp32.argtypes = sig
    lib.attn_fwd_fp32.restype = i32
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


def _stream_handle(device):
    return torch.cuda.current_stream(device).cuda_stream


def forward(q, k, v, scale=None, causal=False, out=None, lse=None):
    """O, LSE for contiguous [B, H, N, d] tensors on one device.

    bf16 tensors use attn_fwd, fp32 tensors attn_fwd_fp32.  ``scale``
    defaults to 1/sqrt(d).  ``out`` and ``lse`` may be given to reuse buffers.
    Launches on torch's current stream and returns without synchronising.
    """
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share one dtype")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"unsupported dtype {q.dtype}; use bfloat16 or float32")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one 4-D shape [B, H, N, d]")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, N, d]")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must live on one GPU")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    fn = attn_fwd if q.dtype == torch.bfloat16 else attn_fwd_fp32
    with torch.cuda.device(q.device):
        fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
           B, H, N, d, scale, causal, _stream_handle(q.device))
    return out, lse
