"""GPU parity of the FP8 (E4M3) forward pass (fa_fwd_fp8, through the C ABI).

Seeded E4M3 inputs (fp32 normal draws rounded to nearest E4M3); the fp64
oracle sees exactly the stored values times the descale factors.  O is bf16.

Tolerance, per element, from the arithmetic of the kernel:
  * q . k products of E4M3 values are exact in fp32 and summed in fp32, so
    the scores, the exp2 weights P~ (fp32) and lse carry only fp32 rounding;
    lse is held to 1e-3 as in the 16-bit paths;
  * each weight P~_j is rounded to E4M3 before the P V product: a relative
    error up to 2^-4 in E4M3's normal range, which bounds the output error by
    2^-4 * sum_j p_ij |v_j| (the oracle's output for |V|, "O_abs");
  * weights below 2^-6 (relative to the kernel's running reference) fall in
    E4M3's subnormal range, where the error is at most 2^-10 per weight in
    absolute terms; these errors have random signs, and an absolute floor of
    2^-7 covers them at the sizes tested (measured worst cases are printed);
  * O is rounded once to bf16: half an ulp.
"""
import math

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.test_gpu_parity import GUARD, _host_widen, _torch, half_ulp

pytestmark = pytest.mark.gpu


def run_fp8(q, k, v, scale, qd, kd, vd, causal):
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    B, H, N, D = q.shape
    n_o, n_l = B * H * N * D, B * H * N
    o_buf = torch.full((n_o + GUARD,), float("nan"), dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((n_l + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    o_buf[n_o:] = 7.0
    l_buf[n_l:] = -3.0
    wsb = fa.fa_fwd_fp8_workspace_bytes(B, H, N, D)
    ws = torch.full((wsb + 64 * GUARD,), 0x7F, dtype=torch.uint8, device="cuda")  # NaN codes
    dq, dk, dv = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in (q, k, v))
    print("fa_fwd_fp8 B%d H%d N%d D%d causal=%d scale=%g descale=(%g,%g,%g)" % (B, H, N, D, causal, scale, qd,
                                                                                kd, vd), flush=True)
    st = fa.fa_fwd_fp8(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), o_buf.data_ptr(), l_buf.data_ptr(), B, H, N, D,
                       float(scale), float(qd), float(kd), float(vd), int(causal), ws.data_ptr(), wsb,
                       torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    assert torch.all(o_buf[n_o:] == 7.0) and torch.all(l_buf[n_l:] == -3.0), "output guard band overwritten"
    assert torch.all(ws[wsb:] == 0x7F), "workspace guard band overwritten"
    o = o_buf[:n_o].view(B, H, N, D)
    lse = l_buf[:n_l].view(B, H, N)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), "unwritten or non-finite outputs"
    return o, lse


def check_fp8(B, H, N, D, causal, seed, scale=None, descale=(1.0, 1.0, 1.0), n_rows=None, slices=None):
    q, k, v = fi.make_qkv(B, H, N, D, "e4m3", seed)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    qd, kd, vd = descale
    o, lse = run_fp8(q, k, v, scale, qd, kd, vd, causal)
    sc = oracle.gpu_scale(scale)
    f32 = lambda x: float(np.float32(x))
    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    worst = ratio = 0.0
    worst_l = 0.0
    for (b, h) in slices:
        rows = np.arange(N, dtype=np.int64) if n_rows is None else fi.sample_rows(N, n_rows, seed=seed + b + h)
        qw = oracle.widen(q[b, h][rows], "e4m3") * f32(qd)
        kw = oracle.widen(k[b, h], "e4m3") * f32(kd)
        vw = oracle.widen(v[b, h], "e4m3") * f32(vd)
        o_ref, l_ref = oracle.attention_rows(qw, kw, vw, rows, sc, causal)
        o_abs, _ = oracle.attention_rows(qw, kw, np.abs(vw), rows, sc, causal)
        o_got = _host_widen(o[b, h][torch_idx(rows)], "bf16")
        l_got = lse[b, h][torch_idx(rows)].cpu().numpy().astype(np.float64)
        err = np.abs(o_got - o_ref)
        tol = 2.0 ** -4 * o_abs + 2.0 ** -7 + half_ulp(o_ref, "bf16")
        assert (err <= tol).all(), (float(err.max()), float((err / tol).max()))
        worst = max(worst, float(err.max()))
        ratio = max(ratio, float((err / (2.0 ** -4 * o_abs + 1e-30)).max()))
        worst_l = max(worst_l, float(np.abs(l_got - l_ref).max()))
    print("  max|dO|=%.3g  max |dO| / (2^-4 O_abs)=%.3g  max|dlse|=%.3g" % (worst, ratio, worst_l), flush=True)
    assert worst_l <= 1e-3


def torch_idx(rows):
    torch = _torch()
    return torch.from_numpy(np.asarray(rows, dtype=np.int64)).to("cuda")


@pytest.mark.parametrize("N", [1, 100, 128, 129, 300, 1000])
@pytest.mark.parametrize("D", [32, 64, 96, 128, 160, 192, 224, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ragged(N, D, causal):
    check_fp8(2, 3, N, D, causal, seed=900 + N + D)


@pytest.mark.parametrize("D", [32, 96, 160, 192, 224, 256])
def test_fp8_head_dims_descales(D):
    """The head dims beyond 64/128 with non-unit descales and a negative scale."""
    for causal in (False, True):
        check_fp8(1, 2, 700, D, causal, seed=970 + D, scale=-0.7 / math.sqrt(D), descale=(0.5, 2.0, 1.5))


@pytest.mark.parametrize("D", [32, 96, 160, 192, 224, 256])
def test_fp8_head_dims_sampled(D):
    """B4 H8 N4096 at each added head dim: 96 sampled rows of 6 seeded slices."""
    slices = fi.sample_slices(4, 8, 6, seed=17)
    for causal in (False, True):
        check_fp8(4, 8, 4096, D, causal, seed=1010 + D, n_rows=96, slices=slices)


@pytest.mark.parametrize("descale", [(0.5, 2.0, 1.0), (0.25, 0.125, 3.0), (-1.0, 1.0, 0.5)])
def test_fp8_descales(descale):
    for causal in (False, True):
        check_fp8(1, 2, 500, 128, causal, seed=950, descale=descale)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_headline_sampled(causal):
    """The headline shape in FP8 (B4 H16 N4096 D128): 128 sampled rows of 8 seeded slices."""
    slices = fi.sample_slices(4, 16, 8, seed=16)
    check_fp8(4, 16, 4096, 128, causal, seed=1004, n_rows=128, slices=slices)


def test_fp8_binding():
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    q, k, v = fi.make_qkv(1, 2, 333, 128, "e4m3", seed=960)
    o1, l1 = run_fp8(q, k, v, 0.09, 1.0, 1.0, 1.0, True)
    dq, dk, dv = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in (q, k, v))
    o2, l2 = fa.fwd_fp8(dq, dk, dv, scale=0.09, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
