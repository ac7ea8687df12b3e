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

It also holds the merge of key-split partial results (``lse_merge``), in
numpy fp64, written from the pages' online-softmax merge step.
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
        lib.oracle_attention_rows_range.restype = ctypes.c_int
        lib.oracle_attention_rows_range.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_attention_rows_general.restype = ctypes.c_int
        lib.oracle_attention_rows_general.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int,
        ]
        lib.oracle_attention_bwd.restype = ctypes.c_int
        lib.oracle_attention_bwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
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
    dtype 'e4m3': the array holds OCP FP8 E4M3 codes (uint8).
    """
    if dtype == "bf16":
        bits = np.ascontiguousarray(x).view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "e4m3":
        # OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
        # field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities
        b = np.ascontiguousarray(x).view(np.uint8).astype(np.int64)
        e, m = (b >> 3) & 15, b & 7
        mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
        return np.where(b & 0x80, -mag, mag)
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


def attention_rows(q_rows, k, v, rows, scale: float, causal: bool, n_threads: int = 0,
                   key_range=None, causal_offset=None):
    """One [N, D] slice: outputs (O_rows [R, D], lse_rows [R]) in fp64 for the query
    positions ``rows`` (q_rows[r] is query rows[r]).  All arrays are float64.

    ``key_range = (lo, hi)`` restricts the keys to lo <= j < hi (the partial
    result of one key split); a row with no visible key gets lse = -inf and
    O = 0.  ``causal_offset`` (n_keys - n_queries) switches to a slice whose
    query count differs from its key count: causal query i then sees keys
    j <= i + causal_offset (bottom-right alignment); None means square."""
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
    lo, hi = (0, n_keys) if key_range is None else (int(key_range[0]), int(key_range[1]))
    if causal_offset is None:
        rc = lib.oracle_attention_rows_range(
            q_rows.ctypes.data, k.ctypes.data, v.ctypes.data, n_keys, d,
            rows.ctypes.data, rows.shape[0], lo, hi, float(scale), int(bool(causal)),
            o.ctypes.data, lse.ctypes.data, int(n_threads))
    else:
        rc = lib.oracle_attention_rows_general(
            q_rows.ctypes.data, k.ctypes.data, v.ctypes.data, n_keys, d,
            rows.ctypes.data, rows.shape[0], lo, hi, float(scale), int(bool(causal)),
            int(causal_offset), o.ctypes.data, lse.ctypes.data, int(n_threads))
    if rc != 0:
        raise ValueError("oracle_attention_rows failed with code %d" % rc)
    return o, lse


def attention(q, k, v, scale: float, causal: bool, n_threads: int = 0, key_range=None):
    """Full [..., N, D] tensors in fp64 (leading dims are independent slices).
    Returns (O [..., N, D], lse [..., N]) in fp64.  ``key_range`` as in
    ``attention_rows``."""
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
        o[s], lse[s] = attention_rows(qf[s], kf[s], vf[s], rows, scale, causal, n_threads,
                                      key_range)
    return o.reshape(*lead, n, d), lse.reshape(*lead, n)


def attention_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool, n_threads: int = 0,
                     seqs=None, rows_of=None):
    """Packed variable-length sequences, head-major: q [H, total_q, D], k and v
    [H, total_k, D]; sequence b holds query rows cu_q[b]..cu_q[b+1]-1 and key rows
    cu_k[b]..cu_k[b+1]-1 of every head.  Each (sequence, head) is one slice with
    n_q = cu_q[b+1] - cu_q[b] queries and n_k keys, causal aligned bottom-right
    (query i sees keys j <= i + n_k - n_q); a row that sees no key gets lse = -inf
    and O = 0, as does every row of a sequence with no keys.

    ``seqs`` limits the work to some sequences and ``rows_of(b)`` to some rows of
    each (positions within the sequence).  Returns a list of
    (b, rows, O [H, R, D], lse [H, R]) in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    H, _, d = q.shape
    out = []
    for b in (range(len(cu_q) - 1) if seqs is None else seqs):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        rows = np.arange(q1 - q0, dtype=np.int64) if rows_of is None else np.asarray(rows_of(b), np.int64)
        o = np.zeros((H, rows.size, d))
        lse = np.full((H, rows.size), -np.inf)
        if k1 > k0 and rows.size:
            for h in range(H):
                o[h], lse[h] = attention_rows(q[h, q0 + rows], k[h, k0:k1], v[h, k0:k1], rows, scale,
                                              causal, n_threads, causal_offset=(k1 - k0) - (q1 - q0))
        out.append((b, rows, o, lse))
    return out


def attention_bwd(q, k, v, dout, scale: float, causal: bool, n_threads: int = 0):
    """Gradients (dQ, dK, dV) in fp64 of the square attention forward for the
    output gradient dout; [..., N, D] arrays, leading dims independent slices.
    The definition (explicit P, softmax Jacobian) is in oracle.c."""
    lib = _load()
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    if not (q.shape == k.shape == v.shape == dout.shape) or q.ndim < 2:
        raise ValueError("q, k, v, dout must share one [..., N, D] shape")
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    flat = [np.ascontiguousarray(x.reshape(-1, n, d)) for x in (q, k, v, dout)]
    outs = [np.empty_like(flat[0]) for _ in range(3)]
    for s in range(flat[0].shape[0]):
        rc = lib.oracle_attention_bwd(flat[0][s].ctypes.data, flat[1][s].ctypes.data, flat[2][s].ctypes.data,
                                      flat[3][s].ctypes.data, n, d, float(scale), int(bool(causal)),
                                      outs[0][s].ctypes.data, outs[1][s].ctypes.data, outs[2][s].ctypes.data,
                                      int(n_threads))
        if rc != 0:
            raise ValueError("oracle_attention_bwd failed with code %d" % rc)
    return tuple(x.reshape(*lead, n, d) for x in outs)


def lse_merge(part_o, part_lse):
    """Merge partial results over disjoint key sets into the result over their union.

    part_o [P, ..., D] and part_lse [P, ...] (fp64): part p is the normalised
    output O_p and logsumexp lse_p of the same query rows over key set p.
    This is the online-softmax merge of a running state with a new block's
    statistics (KingOfEgg's FlashAttention v1 post, section 4.3, the
    m_new / l_new / O update), applied to P parts at once.  A part's
    (m_p, l_p) pair enters only through lse_p = m_p + ln l_p, so each part
    is taken with m_p = lse_p and l_p = 1:

        m   = max_p lse_p
        w_p = exp(lse_p - m)          (the exp(m_old - m_new) factors)
        l   = sum_p w_p
        O   = sum_p w_p O_p / l
        lse = m + ln l

    A part with lse_p = -inf (no visible key) has weight 0 and its O_p is
    not read.  A row whose parts are all -inf gets lse = -inf and O = 0.
    Returns (O [..., D], lse [...]) in fp64.
    """
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    if part_o.shape[:-1] != part_lse.shape or part_lse.ndim < 1 or part_lse.shape[0] < 1:
        raise ValueError("part_o %s and part_lse %s do not match" % (part_o.shape, part_lse.shape))
    m = part_lse.max(axis=0)
    empty = m == -np.inf
    m_safe = np.where(empty, 0.0, m)
    w = np.where(part_lse == -np.inf, 0.0, np.exp(part_lse - m_safe))
    l = w.sum(axis=0)
    contrib = np.where((w > 0)[..., None], w[..., None] * np.nan_to_num(part_o), 0.0)
    o = np.where(empty[..., None], 0.0, contrib.sum(axis=0) / np.where(empty, 1.0, l)[..., None])
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return o, lse
