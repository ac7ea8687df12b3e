"""libfa: exact, tiled attention forward pass for MI355X (gfx950).

Thin ctypes binding over the C ABI declared in ``include/fa.h``.  Every step
of the computation runs in the HIP kernels of ``libfa.so``; this module only
marshals arguments.  There is no fallback: if the library is missing or the
device is not gfx950 the calls raise.

Names follow the C ABI: ``fa_fwd``, ``fa_check_args``, ``fa_status_string``,
``fa_abi_version``.  ``fwd`` is a convenience wrapper that allocates O and lse
with torch (device memory and the current stream are all torch provides).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["FA_DTYPE_F32", "FA_DTYPE_BF16", "FA_DTYPE_F16", "FA_OK", "FA_ERR_INVALID_ARG",
           "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FaError", "lib_path", "load_library", "fa_fwd",
           "fa_check_args", "fa_status_string", "fa_abi_version", "fwd"]

FA_DTYPE_F32, FA_DTYPE_BF16, FA_DTYPE_F16 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3

_PKG = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib_path() -> str:
    return os.path.join(_PKG, "libfa.so")


class FaError(RuntimeError):
    def __init__(self, status: int, what: str = "fa_fwd"):
        self.status = status
        super().__init__("%s failed: status %d (%s)" % (what, status, fa_status_string(status)))


def load_library():
    """Load libfa.so from the package directory; raise if it has not been built."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError("libfa.so is not built (expected at %s); run "
                              "`python -c 'import __graft_entry__ as g; g.build()'`" % path)
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.fa_fwd.restype = ctypes.c_int
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                               ctypes.c_int, ctypes.c_int, vp]
        lib.fa_check_args.restype = ctypes.c_int
        lib.fa_check_args.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_char_p]
        lib.fa_status_string.restype = ctypes.c_char_p
        lib.fa_status_string.argtypes = [ctypes.c_int]
        lib.fa_abi_version.restype = ctypes.c_int
        lib.fa_abi_version.argtypes = []
        _lib = lib
    return _lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_abi_version() -> int:
    return int(load_library().fa_abi_version())


def fa_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, D: int,
           scale: float, causal: int, dtype: int, stream: int) -> int:
    """Raw C call with integer device addresses; returns the fa_status code."""
    return int(load_library().fa_fwd(q, k, v, o, lse, B, H, N, D, scale, causal, dtype, stream))


def fa_check_args(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, D: int,
                  scale: float, causal: int, dtype: int, arch: str | None = None) -> int:
    """Host-only argument check (no HIP call); returns the fa_status code."""
    a = arch.encode() if arch is not None else None
    return int(load_library().fa_check_args(q, k, v, o, lse, B, H, N, D, scale, causal, dtype, a))


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FA_DTYPE_F32, torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_F16}
    if t not in codes:
        raise TypeError("unsupported dtype %s (float32, bfloat16, float16)" % (t,))
    return codes[t]


def fwd(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None, stream=None):
    """O, lse = softmax(scale * Q K^T) V for [B, H, N, D] CUDA tensors (torch, on a gfx950 device).

    scale defaults to 1/sqrt(D).  O has q's dtype; lse is float32 [B, H, N].
    Enqueued on ``stream`` (default: torch's current stream); returns without
    synchronising.
    """
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, N, D] with the same shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError("%s is not a device tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous [B, H, N, D]" % name)
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, N, D, float(scale), int(bool(causal)), _dtype_code(q.dtype), handle)
    if st != FA_OK:
        raise FaError(st)
    return out, lse
