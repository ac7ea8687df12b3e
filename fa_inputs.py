"""Seeded synthetic inputs for the attention forward pass.

Shared by both sides of every parity check (the HIP path and the fp64
oracle) and by the benchmark.  It holds none of the method's arithmetic:
only random draws, rounding of the draws to the storage type, row sampling
and the workload table.

Recipe (stated once, used everywhere):
  * numpy ``Generator(PCG64)``; the three tensors Q, K, V get the streams
    ``SeedSequence(seed).spawn(3)`` in that order;
  * each element is ``standard_normal(dtype=float32) * sigma``;
  * for bf16 / fp16 storage the fp32 draw is rounded to nearest-even
    (bf16 kept as its 16-bit pattern, a uint16 array); for FP8 E4M3 storage
    it is rounded to the nearest E4M3 value (ties to even, saturating at
    448), kept as uint8 codes.
"""
from __future__ import annotations

import numpy as np

DTYPES = ("f32", "bf16", "f16", "e4m3")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns.
    NaN stays NaN (quiet), infinities stay infinities."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def _e4m3_magnitudes() -> np.ndarray:
    """Values of the 127 non-negative finite OCP FP8 E4M3 codes 0x00..0x7E, by code."""
    codes = np.arange(127)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
    no infinities): nearest value, ties to the even code, magnitudes beyond 448
    saturate to 448.  Returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    mags = _e4m3_magnitudes()
    a = np.minimum(np.abs(x), mags[-1])
    hi = np.clip(np.searchsorted(mags, a, side="left"), 1, len(mags) - 1)
    lo = hi - 1
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a == mags[hi], hi, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw(rng: np.random.Generator, shape, sigma: float, dtype: str, chunk: int = 1 << 24):
    n = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
    elif dtype == "f16":
        out = np.empty(n, dtype=np.float16)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
    elif dtype == "e4m3":
        out = np.empty(n, dtype=np.uint8)
    else:
        raise ValueError(dtype)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        if dtype == "f32":
            out[s:e] = x
        elif dtype == "f16":
            out[s:e] = x.astype(np.float16)  # numpy rounds to nearest-even
        elif dtype == "e4m3":
            out[s:e] = f32_to_e4m3_bits(x)
        else:
            out[s:e] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def make_qkv(B: int, H: int, N: int, D: int, dtype: str, seed: int,
             sigma_q: float = 1.0, sigma_k: float = 1.0, sigma_v: float = 1.0):
    """Q, K, V of shape [B, H, N, D] in storage form (float32, float16 or bf16 bits)."""
    ss = np.random.SeedSequence(seed).spawn(3)
    shape = (B, H, N, D)
    q = _draw(np.random.Generator(np.random.PCG64(ss[0])), shape, sigma_q, dtype)
    k = _draw(np.random.Generator(np.random.PCG64(ss[1])), shape, sigma_k, dtype)
    v = _draw(np.random.Generator(np.random.PCG64(ss[2])), shape, sigma_v, dtype)
    return q, k, v


def make_seqlens(n_seqs: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Sequence lengths for a packed batch: n_seqs integers drawn uniformly from
    [lo, hi] (PCG64 seeded with ``seed``)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi, size=n_seqs, endpoint=True).astype(np.int64)


def cu_seqlens(lens) -> np.ndarray:
    """Start row of every sequence plus the total: [0, l0, l0 + l1, ...] (int32)."""
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


def make_packed(H: int, total_q: int, total_k: int, D: int, dtype: str, seed: int,
                sigma_q: float = 1.0, sigma_k: float = 1.0, sigma_v: float = 1.0):
    """Head-major packed Q [H, total_q, D], K and V [H, total_k, D], drawn like make_qkv."""
    ss = np.random.SeedSequence(seed).spawn(3)
    q = _draw(np.random.Generator(np.random.PCG64(ss[0])), (H, total_q, D), sigma_q, dtype)
    k = _draw(np.random.Generator(np.random.PCG64(ss[1])), (H, total_k, D), sigma_k, dtype)
    v = _draw(np.random.Generator(np.random.PCG64(ss[2])), (H, total_k, D), sigma_v, dtype)
    return q, k, v


def sample_rows(N: int, n_rows: int, seed: int) -> np.ndarray:
    """Sorted query positions: 0 and N-1 always, the rest drawn without replacement."""
    if n_rows >= N:
        return np.arange(N, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = {0, N - 1}
    rest = rng.choice(np.arange(1, N - 1), size=max(0, n_rows - len(fixed)), replace=False)
    return np.array(sorted(fixed.union(int(r) for r in rest)), dtype=np.int64)


def sample_slices(B: int, H: int, n: int, seed: int):
    """n distinct (b, h) pairs drawn without replacement, sorted."""
    rng = np.random.Generator(np.random.PCG64(seed))
    flat = rng.choice(B * H, size=min(n, B * H), replace=False)
    return [(int(f) // H, int(f) % H) for f in sorted(flat)]


# The five synthetic workloads.  "check" says which query rows the oracle
# evaluates: "full" (every row of every slice), or ("rows", n) per slice, or
# ("slices_rows", n_slices, n_rows).
WORKLOADS = {
    "tiny_f32": dict(B=1, H=1, N=128, D=64, dtype="f32", modes=(False,), seed=1001,
                     sigma=(1.0, 1.0, 1.0), check=("full",)),
    "small_bf16": dict(B=2, H=8, N=1024, D=64, dtype="bf16", modes=(False, True), seed=1002,
                       sigma=(1.0, 1.0, 1.0), check=("full",)),
    "small_f32": dict(B=2, H=8, N=1024, D=64, dtype="f32", modes=(False, True), seed=1003,
                      sigma=(1.0, 1.0, 1.0), check=("full",)),
    "headline_bf16": dict(B=4, H=16, N=4096, D=128, dtype="bf16", modes=(False, True), seed=1004,
                          sigma=(1.0, 1.0, 1.0), check=("rows", 256)),
    "wide_bf16": dict(B=32, H=32, N=4096, D=64, dtype="bf16", modes=(False,), seed=1005,
                      sigma=(1.0, 1.0, 1.0), check=("slices_rows", 8, 128)),
    "long_causal_bf16": dict(B=1, H=8, N=131072, D=128, dtype="bf16", modes=(True,), seed=1006,
                             sigma=(0.5, 0.5, 1.0), check=("rows", 64)),
}


# Packed variable-length batch: 16 sequences of lengths drawn uniformly from
# [128, 4096] (self-attention, n_q = n_k per sequence), 16 heads, D = 128.
VARLEN_WORKLOAD = dict(n_seqs=16, lo=128, hi=4096, H=16, D=128, dtype="bf16", seed=1007,
                       sigma=(1.0, 1.0, 1.0))


def workload_flops(B: int, H: int, N: int, D: int, causal: bool) -> float:
    """The metric's FLOP count: 4*B*H*N^2*D, halved for causal."""
    f = 4.0 * B * H * N * N * D
    return f / 2 if causal else f


def varlen_flops(lens_q, lens_k, H: int, D: int, causal: bool) -> float:
    """4*H*D*sum_b n_q(b)*n_k(b), halved for causal (the dense metric's convention)."""
    f = 4.0 * H * D * float(np.sum(np.asarray(lens_q, np.float64) * np.asarray(lens_k, np.float64)))
    return f / 2 if causal else f
