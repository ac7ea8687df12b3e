"""CPU tests of the seeded input generator (no method arithmetic lives there)."""
import numpy as np
import torch

import fa_inputs as fi
import oracle


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40, np.inf, -np.inf],
                 dtype=np.float32),
        # exact ties: mantissa low half 0x8000 with even and odd upper parts
        np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32).view(np.float32),
    ])
    got = fi.f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    nan = fi.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(fi.bf16_bits_to_f32(nan))[0]


def test_generator_is_seeded_and_shaped():
    a = fi.make_qkv(1, 2, 33, 64, "bf16", seed=7)
    b = fi.make_qkv(1, 2, 33, 64, "bf16", seed=7)
    c = fi.make_qkv(1, 2, 33, 64, "bf16", seed=8)
    for x, y in zip(a, b):
        assert x.shape == (1, 2, 33, 64) and x.dtype == np.uint16 and np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    # Q, K, V come from different streams
    assert not np.array_equal(a[0], a[1])
    f = fi.make_qkv(1, 1, 64, 64, "f32", seed=7, sigma_q=0.5)
    g = fi.make_qkv(1, 1, 64, 64, "f32", seed=7)
    assert np.array_equal(f[0], g[0] * np.float32(0.5))
    h = fi.make_qkv(1, 1, 64, 64, "f16", seed=7)
    assert h[0].dtype == np.float16 and np.array_equal(h[0], g[0].astype(np.float16))


def test_sample_rows_and_slices():
    r = fi.sample_rows(4096, 256, seed=5)
    assert r.size == 256 and r[0] == 0 and r[-1] == 4095 and np.all(np.diff(r) > 0)
    assert np.array_equal(fi.sample_rows(10, 64, seed=5), np.arange(10))
    s = fi.sample_slices(32, 32, 8, seed=5)
    assert len(set(s)) == 8 and all(0 <= b < 32 and 0 <= h < 32 for b, h in s)


def test_workload_table():
    w = fi.WORKLOADS["headline_bf16"]
    assert (w["B"], w["H"], w["N"], w["D"], w["dtype"]) == (4, 16, 4096, 128, "bf16")
    assert fi.workload_flops(4, 16, 4096, 128, False) == 549755813888.0
    assert fi.workload_flops(4, 16, 4096, 128, True) == 549755813888.0 / 2


def test_e4m3_decode_fixed_points():
    """OCP FP8 E4M3 code points: 1.0 = 0 0111 000, the largest normal 448 =
    0 1111 110, the smallest normal 2^-6 = 0 0001 000, the smallest subnormal
    2^-9 = 0 0000 001, NaN = S 1111 111, and the sign bit."""
    codes = np.array([0x38, 0x7E, 0x08, 0x01, 0x00, 0xB8, 0x40, 0x3C, 0x07], dtype=np.uint8)
    want = np.array([1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 0.0, -1.0, 2.0, 1.5, 7 * 2.0 ** -9])
    assert np.array_equal(oracle.widen(codes, "e4m3"), want)
    assert np.isnan(oracle.widen(np.array([0x7F, 0xFF], dtype=np.uint8), "e4m3")).all()


def test_e4m3_round_trip_and_rounding():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.widen(codes, "e4m3")
    assert np.array_equal(fi.f32_to_e4m3_bits(vals), codes)
    # midpoints round to the even code; beyond 448 saturates
    mid = (vals[(codes >= 0x08) & (codes < 0x7E)] + oracle.widen(codes[(codes >= 0x08) & (codes < 0x7E)] + 1, "e4m3")) / 2
    got = fi.f32_to_e4m3_bits(mid)
    assert np.all(got % 2 == 0)
    assert list(fi.f32_to_e4m3_bits(np.array([449.0, 1e6, -1e6]))) == [0x7E, 0x7E, 0xFE]
