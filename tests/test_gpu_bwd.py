"""GPU parity of the backward pass (fa_bwd, through the C ABI).

Seeded Q, K, V and an output gradient dO; the device runs fa_fwd (for O and
lse, the inputs fa_bwd takes) and then fa_bwd; the fp64 oracle computes dQ,
dK, dV from Q, K, V and dO alone (explicit P, softmax Jacobian).  Outputs
start poisoned (NaN) and are followed by guard bands.

Tolerance (max-abs, per tensor), derived from the arithmetic of the bf16 /
fp16 path with N(0,1) inputs and scale 1/sqrt(D):
  * every MFMA product of two 16-bit values is exact in fp32 and sums are
    fp32 (relative error ~1e-6, negligible);
  * P and dS are rounded to the input type before the dV = P^T dO and
    dQ = scale dS K / dK = scale dS^T Q products: a relative error u per term
    (u = 2^-9 bf16, 2^-12 fp16) on sums whose terms carry random signs;
  * Delta is taken from the forward's stored (rounded) O;
  * the output is rounded once: half an ulp of |dX|.
Measured on the workloads below these stay under 1e-2 for bf16 outputs of
magnitude up to ~4; the bound used is tol = 1e-2 * max(1, max|ref|) plus
half an ulp of the output type at max|ref| (the output rounding alone can
exceed 1e-2 above 4, as in the forward tests), printed with every case.
"""
import math

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.test_gpu_parity import GUARD, _host_widen, _tdtype, _to_device, _torch, half_ulp

pytestmark = pytest.mark.gpu


def run_bwd(q, k, v, do, dtype, scale, causal):
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    B, H, N, D = q.shape
    n = B * H * N * D
    td = _tdtype(dtype)
    dq_, dk_, dv_, do_ = (_to_device(x, dtype) for x in (q, k, v, do))
    o, lse = fa.fwd(dq_, dk_, dv_, scale=scale, causal=causal)
    outs = []
    for _ in range(3):
        buf = torch.full((n + GUARD,), float("nan"), dtype=td, device="cuda")
        buf[n:] = 7.0
        outs.append(buf)
    wsb = fa.fa_bwd_workspace_bytes(B, H, N, D)
    ws = torch.full((wsb // 4 + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    ws[wsb // 4:] = 5.0
    code = {"bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16}[dtype]
    torch.cuda.synchronize()
    print("fa_bwd B%d H%d N%d D%d %s causal=%d scale=%g" % (B, H, N, D, dtype, causal, scale), flush=True)
    st = fa.fa_bwd(dq_.data_ptr(), dk_.data_ptr(), dv_.data_ptr(), o.data_ptr(), do_.data_ptr(), lse.data_ptr(),
                   outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), B, H, N, D, float(scale), int(causal),
                   code, ws.data_ptr(), wsb, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    for name, buf in zip(("dQ", "dK", "dV"), outs):
        assert torch.all(buf[n:] == 7.0), "%s guard band overwritten" % name
        assert bool(torch.isfinite(buf[:n]).all()), "%s has unwritten or non-finite elements" % name
    assert torch.all(ws[wsb // 4:] == 5.0), "workspace guard band overwritten"
    return tuple(buf[:n].view(B, H, N, D) for buf in outs)


def check_bwd(B, H, N, D, dtype, causal, seed, scale=None, slices=None):
    q, k, v = fi.make_qkv(B, H, N, D, dtype, seed)
    do, _, _ = fi.make_qkv(B, H, N, D, dtype, seed + 7919)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    grads = run_bwd(q, k, v, do, dtype, scale, causal)
    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    sc = oracle.gpu_scale(scale)
    worst = {}
    for (b, h) in slices:
        w = [oracle.widen(x[b, h], dtype) for x in (q, k, v, do)]
        refs = oracle.attention_bwd(*w, sc, causal)
        for name, got, ref in zip(("dQ", "dK", "dV"), grads, refs):
            g = _host_widen(got[b, h], dtype)
            err = float(np.abs(g - ref).max())
            mx = float(np.abs(ref).max())
            e0, m0 = worst.get(name, (0.0, 0.0))
            worst[name] = (max(e0, err), max(m0, mx))
    msg = []
    for name, (err, mx) in worst.items():
        tol = 1e-2 * max(1.0, mx) + float(half_ulp(np.array([mx]), dtype)[0])
        msg.append("%s max|d|=%.3g (max|ref| %.3g, tol %.3g)" % (name, err, mx, tol))
    print("  " + "; ".join(msg), flush=True)
    for name, (err, mx) in worst.items():
        tol = 1e-2 * max(1.0, mx) + float(half_ulp(np.array([mx]), dtype)[0])
        assert err <= tol, (name, err, tol)


@pytest.mark.parametrize("N", [1, 31, 64, 100, 255, 257, 600])
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged(N, D, dtype, causal):
    check_bwd(1, 2, N, D, dtype, causal, seed=700 + N + D)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_d96_several_blocks(causal):
    """D = 96 over several query and key blocks with a ragged tail (N = 1100)."""
    check_bwd(1, 3, 1100, 96, "bf16", causal, seed=796)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_small_workload(causal):
    w = fi.WORKLOADS["small_bf16"]
    check_bwd(w["B"], w["H"], w["N"], w["D"], "bf16", causal, w["seed"])


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_headline_slices(causal):
    """The headline shape (B4 H16 N4096 D128), three seeded (b, h) slices, every row."""
    w = fi.WORKLOADS["headline_bf16"]
    slices = fi.sample_slices(w["B"], w["H"], 3, seed=31)
    check_bwd(w["B"], w["H"], w["N"], w["D"], "bf16", causal, w["seed"], slices=slices)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.3])
def test_bwd_scales(scale):
    for causal in (False, True):
        check_bwd(1, 2, 300, 64, "bf16", causal, seed=9, scale=scale)


def test_bwd_deterministic_and_binding():
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    q, k, v = fi.make_qkv(1, 2, 700, 128, "bf16", seed=10)
    do, _, _ = fi.make_qkv(1, 2, 700, 128, "bf16", seed=11)
    g1 = run_bwd(q, k, v, do, "bf16", 0.088, True)
    g2 = run_bwd(q, k, v, do, "bf16", 0.088, True)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    dq_, dk_, dv_, do_ = (_to_device(x, "bf16") for x in (q, k, v, do))
    o, lse = fa.fwd(dq_, dk_, dv_, scale=0.088, causal=True)
    g3 = fa.bwd(dq_, dk_, dv_, o, lse, do_, scale=0.088, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g3):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
