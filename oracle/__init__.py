"""fp64 CPU oracle for the exact attention forward pass (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path (the
HIP library and its Python binding) never imports this package, and this
package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain definition of softmax(scale *
Q K^T) V with an explicit score row and a three-pass softmax, see that
file's header for the passages it follows).  This module only

  * widens stored inputs to fp64 (exact for fp32, fp16 and bf16 bit
    patterns),
  * rounds the scale to the fp32 value a GPU caller passes
    (``float(np.float32(scale))``), and
  * loops over (batch, head) slices, handing each to the C routine.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (fp64, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_attention_rows.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_default_threads.restype = ctypes.c_int
        lib.oracle_default_threads.argtypes = []
        _lib = lib
    return _lib


def default_threads() -> int:
    return int(_load().oracle_default_threads())


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64.

    dtype 'f32' / 'f16': the array holds those floats.
    dtype 'bf16': the array holds the 16-bit patterns (uint16); a bf16 value
    is the fp32 value whose upper 16 bits are the pattern.
    """
    if dtype == "bf16":
        bits = np.ascontiguousarray(x).view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError("unknown dtype %r" % (dtype,))


def gpu_scale(scale: float) -> float:
    """The scale as the fp32 value handed to the device, widened back to fp64."""
    return float(np.float32(scale))


def attention_rows(q_rows, k, v, rows, scale: float, causal: bool, n_threads: int = 0):
    """One [N, D] slice: outputs (O_rows [R, D], lse_rows [R]) in fp64 for the query
    positions ``rows`` (q_rows[r] is query rows[r]).  All arrays are float64."""
    lib = _load()
    q_rows = np.ascontiguousarray(q_rows, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n_keys, d = k.shape
    if v.shape != (n_keys, d) or q_rows.shape != (rows.shape[0], d):
        raise ValueError("shape mismatch: q_rows %s k %s v %s rows %s"
                         % (q_rows.shape, k.shape, v.shape, rows.shape))
    o = np.empty((rows.shape[0], d), dtype=np.float64)
    lse = np.empty((rows.shape[0],), dtype=np.float64)
    rc = lib.oracle_attention_rows(
        q_rows.ctypes.data, k.ctypes.data, v.ctypes.data, n_keys, d,
        rows.ctypes.data, rows.shape[0], float(scale), int(bool(causal)),
        o.ctypes.data, lse.ctypes.data, int(n_threads))
    if rc != 0:
        raise ValueError("oracle_attention_rows failed with code %d" % rc)
    return o, lse


def attention(q, k, v, scale: float, causal: bool, n_threads: int = 0):
    """Full [..., N, D] tensors in fp64 (leading dims are independent slices).
    Returns (O [..., N, D], lse [..., N]) in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    qf = q.reshape(-1, n, d)
    kf = k.reshape(-1, n, d)
    vf = v.reshape(-1, n, d)
    o = np.empty_like(qf)
    lse = np.empty(qf.shape[:2], dtype=np.float64)
    rows = np.arange(n, dtype=np.int64)
    for s in range(qf.shape[0]):
        o[s], lse[s] = attention_rows(qf[s], kf[s], vf[s], rows, scale, causal, n_threads)
    return o.reshape(*lead, n, d), lse.reshape(*lead, n)
