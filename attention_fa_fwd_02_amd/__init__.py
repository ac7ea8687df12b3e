"""libfa: exact, tiled attention forward pass for MI355X (gfx950).

Thin ctypes binding over the C ABI declared in ``include/fa.h``.  Every step
of the computation runs in the HIP kernels of ``libfa.so``; this module only
marshals arguments.  There is no fallback: if the library is missing or the
device is not gfx950 the calls raise.

Names follow the C ABI: ``fa_fwd``, ``fa_check_args``, ``fa_fwd_split``, ``fa_fwd_split_static``,
``fa_fwd_split_workspace_bytes``, ``fa_fwd_split_choose``, ``fa_lse_merge``,
``fa_fwd_varlen``, ``fa_check_varlen_args``, ``fa_bwd``,
``fa_bwd_workspace_bytes``, ``fa_check_bwd_args``, ``fa_fwd_fp8``,
``fa_fwd_fp8_workspace_bytes``, ``fa_check_fp8_args``, ``fa_fwd_kernel_name``,
``fa_status_string``,
``fa_abi_version``.  ``fwd``, ``fwd_split``, ``fwd_varlen``, ``bwd``,
``fwd_fp8`` and ``lse_merge`` are convenience wrappers that allocate outputs (and
workspaces) with torch (device memory and the current stream are all torch
provides).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["FA_DTYPE_F32", "FA_DTYPE_BF16", "FA_DTYPE_F16", "FA_OK", "FA_ERR_INVALID_ARG",
           "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_MAX_SPLITS", "FaError", "lib_path",
           "load_library", "fa_fwd", "fa_check_args", "fa_fwd_split", "fa_fwd_split_static",
           "fa_fwd_split_workspace_bytes", "FA_STATIC_SCRATCH_BYTES",
           "fa_fwd_split_choose", "fa_lse_merge", "fa_fwd_varlen", "fa_check_varlen_args",
           "fa_bwd", "fa_bwd_workspace_bytes", "fa_check_bwd_args", "fa_fwd_fp8",
           "fa_fwd_fp8_workspace_bytes", "fa_check_fp8_args", "fa_fwd_kernel_name", "fa_status_string",
           "fa_abi_version", "fwd", "fwd_split", "fwd_varlen", "bwd", "fwd_fp8", "lse_merge"]

FA_DTYPE_F32, FA_DTYPE_BF16, FA_DTYPE_F16 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_MAX_SPLITS = 64
FA_STATIC_SCRATCH_BYTES = 64 << 20

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
        lib.fa_fwd_split.restype = ctypes.c_int
        lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                     ctypes.c_int, ctypes.c_int, i64, vp, ctypes.c_uint64, vp]
        lib.fa_fwd_split_static.restype = ctypes.c_int
        lib.fa_fwd_split_static.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                            ctypes.c_int, ctypes.c_int, i64, vp]
        lib.fa_fwd_split_workspace_bytes.restype = ctypes.c_uint64
        lib.fa_fwd_split_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
        lib.fa_fwd_split_choose.restype = i64
        lib.fa_fwd_split_choose.argtypes = [i64, i64, i64, i64, ctypes.c_int, i64]
        lib.fa_lse_merge.restype = ctypes.c_int
        lib.fa_lse_merge.argtypes = [vp, vp, i64, i64, i64, vp, vp, ctypes.c_int, vp]
        lib.fa_fwd_varlen.restype = ctypes.c_int
        lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                      ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
        lib.fa_check_varlen_args.restype = ctypes.c_int
        lib.fa_check_varlen_args.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                             ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_char_p]
        lib.fa_bwd.restype = ctypes.c_int
        lib.fa_bwd.argtypes = [vp] * 9 + [i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                          vp, ctypes.c_uint64, vp]
        lib.fa_bwd_workspace_bytes.restype = ctypes.c_uint64
        lib.fa_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
        lib.fa_check_bwd_args.restype = ctypes.c_int
        lib.fa_check_bwd_args.argtypes = [vp] * 9 + [i64, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                                                     ctypes.c_int, vp, ctypes.c_uint64, ctypes.c_char_p]
        f32 = ctypes.c_float
        lib.fa_fwd_fp8.restype = ctypes.c_int
        lib.fa_fwd_fp8.argtypes = [vp] * 5 + [i64] * 4 + [f32] * 4 + [ctypes.c_int, vp, ctypes.c_uint64, vp]
        lib.fa_fwd_fp8_workspace_bytes.restype = ctypes.c_uint64
        lib.fa_fwd_fp8_workspace_bytes.argtypes = [i64] * 4
        lib.fa_check_fp8_args.restype = ctypes.c_int
        lib.fa_check_fp8_args.argtypes = [vp] * 5 + [i64] * 4 + [f32] * 4 + [ctypes.c_int, vp, ctypes.c_uint64,
                                                                            ctypes.c_char_p]
        lib.fa_fwd_kernel_name.restype = ctypes.c_char_p
        lib.fa_fwd_kernel_name.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, i64]
        lib.fa_status_string.restype = ctypes.c_char_p
        lib.fa_status_string.argtypes = [ctypes.c_int]
        lib.fa_abi_version.restype = ctypes.c_int
        lib.fa_abi_version.argtypes = []
        _lib = lib
    return _lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_fwd_kernel_name(B: int, H: int, N: int, D: int, causal: int, dtype: int, n_cus: int) -> str:
    """Name of the kernel fa_fwd launches for these sizes ("" if it would reject them); host only."""
    return load_library().fa_fwd_kernel_name(B, H, N, D, int(causal), dtype, n_cus).decode()


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


def fa_fwd_split(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, D: int,
                 scale: float, causal: int, dtype: int, n_splits: int, workspace: int,
                 workspace_bytes: int, stream: int) -> int:
    """Raw C call with integer device addresses; returns the fa_status code."""
    return int(load_library().fa_fwd_split(q, k, v, o, lse, B, H, N, D, scale, causal, dtype,
                                           n_splits, workspace, workspace_bytes, stream))


def fa_fwd_split_static(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, D: int,
                        scale: float, causal: int, dtype: int, n_splits: int, stream: int) -> int:
    """Raw C call (split partials in the library's static device array, no
    workspace argument, no allocation); returns the fa_status code."""
    return int(load_library().fa_fwd_split_static(q, k, v, o, lse, B, H, N, D, scale, causal, dtype,
                                                  n_splits, stream))


def fa_fwd_split_workspace_bytes(B: int, H: int, N: int, D: int, n_splits: int) -> int:
    """Workspace bytes fa_fwd_split needs (0 for invalid arguments); host only."""
    return int(load_library().fa_fwd_split_workspace_bytes(B, H, N, D, n_splits))


def fa_fwd_split_choose(B: int, H: int, N: int, D: int, causal: int, n_cus: int) -> int:
    """The library's split count for a device with n_cus compute units; host only."""
    return int(load_library().fa_fwd_split_choose(B, H, N, D, int(causal), n_cus))


def fa_lse_merge(part_o: int, part_lse: int, n_parts: int, rows: int, D: int, o: int, lse: int,
                 dtype: int, stream: int) -> int:
    """Raw C call with integer device addresses; returns the fa_status code."""
    return int(load_library().fa_lse_merge(part_o, part_lse, n_parts, rows, D, o, lse, dtype, stream))


def fa_fwd_varlen(q: int, k: int, v: int, o: int, lse: int, cu_q: int, cu_k: int, n_seqs: int,
                  H: int, total_q: int, total_k: int, max_seqlen_q: int, D: int, scale: float,
                  causal: int, dtype: int, stream: int) -> int:
    """Raw C call with integer device addresses; returns the fa_status code."""
    return int(load_library().fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, n_seqs, H, total_q, total_k,
                                            max_seqlen_q, D, scale, causal, dtype, stream))


def fa_check_varlen_args(q: int, k: int, v: int, o: int, lse: int, cu_q: int, cu_k: int, n_seqs: int,
                         H: int, total_q: int, total_k: int, max_seqlen_q: int, D: int, scale: float,
                         causal: int, dtype: int, arch: str | None = None) -> int:
    """Host-only argument check of fa_fwd_varlen (no HIP call); returns the fa_status code."""
    a = arch.encode() if arch is not None else None
    return int(load_library().fa_check_varlen_args(q, k, v, o, lse, cu_q, cu_k, n_seqs, H, total_q,
                                                   total_k, max_seqlen_q, D, scale, causal, dtype, a))


def fa_bwd(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int, B: int, H: int,
           N: int, D: int, scale: float, causal: int, dtype: int, workspace: int, workspace_bytes: int,
           stream: int) -> int:
    """Raw C call with integer device addresses; returns the fa_status code."""
    return int(load_library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, D, scale, causal, dtype,
                                     workspace, workspace_bytes, stream))


def fa_bwd_workspace_bytes(B: int, H: int, N: int, D: int) -> int:
    """Workspace bytes fa_bwd needs (0 for invalid arguments); host only."""
    return int(load_library().fa_bwd_workspace_bytes(B, H, N, D))


def fa_check_bwd_args(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int, B: int,
                      H: int, N: int, D: int, scale: float, causal: int, dtype: int, workspace: int,
                      workspace_bytes: int, arch: str | None = None) -> int:
    """Host-only argument check of fa_bwd (no HIP call); returns the fa_status code."""
    a = arch.encode() if arch is not None else None
    return int(load_library().fa_check_bwd_args(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, D, scale, causal,
                                                dtype, workspace, workspace_bytes, a))


def fa_fwd_fp8(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, D: int, scale: float,
               q_descale: float, k_descale: float, v_descale: float, causal: int, workspace: int,
               workspace_bytes: int, stream: int) -> int:
    """Raw C call with integer device addresses; returns the fa_status code."""
    return int(load_library().fa_fwd_fp8(q, k, v, o, lse, B, H, N, D, scale, q_descale, k_descale, v_descale,
                                         causal, workspace, workspace_bytes, stream))


def fa_fwd_fp8_workspace_bytes(B: int, H: int, N: int, D: int) -> int:
    """Workspace bytes fa_fwd_fp8 needs (0 for invalid arguments); host only."""
    return int(load_library().fa_fwd_fp8_workspace_bytes(B, H, N, D))


def fa_check_fp8_args(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, D: int, scale: float,
                      q_descale: float, k_descale: float, v_descale: float, causal: int, workspace: int,
                      workspace_bytes: int, arch: str | None = None) -> int:
    """Host-only argument check of fa_fwd_fp8 (no HIP call); returns the fa_status code."""
    a = arch.encode() if arch is not None else None
    return int(load_library().fa_check_fp8_args(q, k, v, o, lse, B, H, N, D, scale, q_descale, k_descale,
                                                v_descale, causal, workspace, workspace_bytes, a))


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FA_DTYPE_F32, torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_F16}
    if t not in codes:
        raise TypeError("unsupported dtype %s (float32, bfloat16, float16)" % (t,))
    return codes[t]


def _check_out(t, name, shape, dtype, device):
    """A caller-supplied output must be a contiguous device tensor of exactly the
    shape and dtype the kernel writes, on the inputs' device: the library writes
    through its raw pointer."""
    if not t.is_cuda or t.device != device:
        raise ValueError("%s must be a device tensor on %s" % (name, device))
    if t.dtype != dtype:
        raise TypeError("%s must have dtype %s, not %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


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
    else:
        _check_out(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_out(lse, "lse", (B, H, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, N, D, float(scale), int(bool(causal)), _dtype_code(q.dtype), handle)
    if st != FA_OK:
        raise FaError(st)
    return out, lse


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def fwd_split(q, k, v, scale: float | None = None, causal: bool = False, n_splits: int | None = None,
              out=None, lse=None, workspace=None, stream=None):
    """``fwd`` computed as key splits merged on the device (fa_fwd_split).

    n_splits defaults to fa_fwd_split_choose for the device's compute-unit
    count.  ``workspace`` (a uint8 CUDA tensor of at least
    fa_fwd_split_workspace_bytes bytes) is allocated when not given.
    Returns (O, lse, workspace); the workspace holds the per-split fp32
    outputs [n_splits, B, H, N, D] followed by their lse [n_splits, B, H, N].
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
    if n_splits is None:
        n_cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        n_splits = fa_fwd_split_choose(B, H, N, D, int(bool(causal)), n_cus)
    need = fa_fwd_split_workspace_bytes(B, H, N, D, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor on %s" % q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_out(lse, "lse", (B, H, N), torch.float32, q.device)
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H, N, D, float(scale), int(bool(causal)), _dtype_code(q.dtype), n_splits,
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(), handle)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_split")
    return out, lse, workspace


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, scale: float | None = None,
               causal: bool = False, out=None, lse=None, stream=None):
    """Packed variable-length attention (fa_fwd_varlen).

    q [H, total_q, D], k and v [H, total_k, D] CUDA tensors (head-major packing);
    cu_seqlens_q / cu_seqlens_k int32 CUDA tensors [n_seqs + 1]; causal masks are
    aligned at the bottom right.  Returns (O [H, total_q, D], lse [H, total_q]).
    """
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [H, total_q, D] and k, v [H, total_k, D]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not t.is_cuda:
            raise ValueError("%s is not a device tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or t.dim() != 1:
            raise TypeError("%s must be a 1-D int32 tensor" % name)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold n_seqs + 1 >= 2 entries")
    H, total_q, D = q.shape
    total_k = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    else:
        _check_out(lse, "lse", (H, total_q), torch.float32, q.device)
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), cu_seqlens_q.numel() - 1, H,
                           total_q, total_k, int(max_seqlen_q), D, float(scale), int(bool(causal)),
                           _dtype_code(q.dtype), handle)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_varlen")
    return out, lse


def bwd(q, k, v, o, lse, dout, scale: float | None = None, causal: bool = False, stream=None):
    """(dQ, dK, dV) of the forward pass that produced o and lse (fa_bwd); all
    [B, H, N, D] CUDA tensors of one dtype (bfloat16, float16, or float32 at
    D = 64 / 128), lse float32 [B, H, N]."""
    import torch
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must all be [B, H, N, D] with the same shape")
    if any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise TypeError("q, k, v, o, dout must share a dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError("%s is not a device tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    B, H, N, D = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be float32 [B, H, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = fa_bwd_workspace_bytes(B, H, N, D)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, D, float(scale), int(bool(causal)),
                    _dtype_code(q.dtype), ws.data_ptr(), ws.numel(), handle)
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def fwd_fp8(q, k, v, scale: float | None = None, causal: bool = False, q_descale: float = 1.0,
            k_descale: float = 1.0, v_descale: float = 1.0, stream=None):
    """FP8 forward (fa_fwd_fp8): q, k, v are uint8 CUDA tensors [B, H, N, D] of E4M3
    codes; returns (O bf16 [B, H, N, D], lse float32 [B, H, N])."""
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, N, D] with the same shape")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.uint8:
            raise TypeError("%s must hold E4M3 codes as uint8" % name)
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous device tensor" % name)
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    need = fa_fwd_fp8_workspace_bytes(B, H, N, D)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, D,
                        float(scale), float(q_descale), float(k_descale), float(v_descale), int(bool(causal)),
                        ws.data_ptr(), ws.numel(), handle)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")
    return o, lse


def lse_merge(part_o, part_lse, out_dtype=None, out=None, lse=None, stream=None):
    """Merge partial results: part_o fp32 [P, ..., D], part_lse fp32 [P, ...] (CUDA,
    contiguous) -> (O [..., D] of out_dtype (default float32), lse [...] fp32)."""
    import torch
    if part_o.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise TypeError("part_o and part_lse must be float32")
    if part_o.dim() < 2 or tuple(part_o.shape[:-1]) != tuple(part_lse.shape):
        raise ValueError("part_o [P, ..., D] and part_lse [P, ...] do not match")
    for name, t in (("part_o", part_o), ("part_lse", part_lse)):
        if not t.is_cuda:
            raise ValueError("%s is not a device tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    P, D = part_o.shape[0], part_o.shape[-1]
    rows = part_lse.numel() // P
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(part_o.shape[1:], dtype=out_dtype, device=part_o.device)
    else:
        _check_out(out, "out", part_o.shape[1:], out.dtype, part_o.device)
    if lse is None:
        lse = torch.empty(part_lse.shape[1:], dtype=torch.float32, device=part_o.device)
    else:
        _check_out(lse, "lse", part_lse.shape[1:], torch.float32, part_o.device)
    handle = _stream_handle(stream, part_o.device)
    with torch.cuda.device(part_o.device):
        st = fa_lse_merge(part_o.data_ptr(), part_lse.data_ptr(), P, rows, D, out.data_ptr(),
                          lse.data_ptr(), _dtype_code(out.dtype), handle)
    if st != FA_OK:
        raise FaError(st, "fa_lse_merge")
    return out, lse
