"""GPU parity of the backward pass (fa_bwd, through the C ABI).

Seeded Q, K, V and an output gradient dO; the device runs fa_fwd (for O and
lse, the inputs fa_bwd takes) and then fa_bwd; the fp64 oracle computes dQ,
dK, dV from Q, K, V and dO alone (explicit P, softmax Jacobian).  Outputs
start poisoned (NaN) and are followed by guard bands.

Tolerance, per element, derived from the arithmetic of the bf16 / fp16 path:
  * every MFMA product of two 16-bit values is exact in fp32 and sums are
    fp32 (relative error ~1e-6, negligible);
  * P and dS are rounded to the input type before the dV = P^T dO and
    dQ = scale dS K / dK = scale dS^T Q products: a relative error u per term
    (u = 2^-9 bf16, 2^-12 fp16), so an element's error is bounded by u times
    A, the sum of the absolute values of the terms that form it
    (A_dV = |P|^T |dO|, A_dQ = scale |dS| |K|, A_dK = scale |dS|^T |Q|);
  * Delta is taken from the forward's stored O, so the forward's own error
    in O (its test holds it to 1e-2) reaches every dS of the row:
    e_i = |dO_i . (O_gpu,i - O_i)| moves dS_ij by P_ij e_i, i.e. dQ_i by up
    to scale e_i sum_j P_ij |k_j| and dK_j by scale sum_i P_ij e_i |q_i|;
  * the output is rounded once: half an ulp of the element.
The bound used is |dX - ref| <= 1e-2 * max(1, A) + E + half an ulp of |ref|
at every element, E being the propagated forward error above (0 for dV): an
element formed from small terms answers to 1e-2, as the forward's O does,
and one formed from large terms gets the same relative room.

fp32 inputs (the fp32 kernels: every product and intermediate in fp32, no
rounding to a narrower type): the per-term error is that of fp32 products
and sums, about 1e-7 relative, so the bound is 1e-5 * max(1, A) + E, the
fp32 forward's own 1e-5 with the same relative room, and no output rounding
term beyond fp32's.  A and E are
computed in the test from the fp64 P, dP, Delta and O of the definition and
the device's O (only for the bound; the reference values are the oracle's).
The largest error, its bound and the tightest margin are printed per case.
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
    code = {"bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16, "f32": fa.FA_DTYPE_F32}[dtype]
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
    return tuple(buf[:n].view(B, H, N, D) for buf in outs) + (o,)


def check_bwd(B, H, N, D, dtype, causal, seed, scale=None, slices=None):
    q, k, v = fi.make_qkv(B, H, N, D, dtype, seed)
    do, _, _ = fi.make_qkv(B, H, N, D, dtype, seed + 7919)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    *grads, o_dev = run_bwd(q, k, v, do, dtype, scale, causal)
    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    sc = oracle.gpu_scale(scale)
    worst = {}
    for (b, h) in slices:
        w = [oracle.widen(x[b, h], dtype) for x in (q, k, v, do)]
        refs = oracle.attention_bwd(*w, sc, causal)
        amag, prop = term_magnitudes(*w, sc, causal, _host_widen(o_dev[b, h], dtype))
        for name, got, ref, A, E in zip(("dQ", "dK", "dV"), grads, refs, amag, prop):
            g = _host_widen(got[b, h], dtype)
            err = np.abs(g - ref)
            rel = 1e-5 if dtype == "f32" else 1e-2
            tol = rel * np.maximum(1.0, A) + E + half_ulp(np.abs(ref), dtype)
            e0, t0, m0 = worst.get(name, (-1.0, 0.0, np.inf))
            i = int(np.argmax(err))
            if err.flat[i] > e0:
                e0, t0 = float(err.flat[i]), float(tol.flat[i])
            worst[name] = (e0, t0, min(m0, float((tol - err).min())))
    print("  " + "; ".join("%s max|d|=%.3g (its bound %.3g), tightest margin %.3g" % (n, e, t, m)
                           for n, (e, t, m) in worst.items()), flush=True)
    for name, (err, tol, margin) in worst.items():
        assert margin >= 0.0, (name, err, tol, margin)


def term_magnitudes(q, k, v, do, sc, causal, o_dev):
    """Per element, the sum of the absolute values of the terms of dQ, dK and
    dV, and the error the device's O propagates into dQ and dK through Delta
    (fp64, from the definition; used only for the tolerance)."""
    s = sc * (q @ k.T)
    if causal:
        n = s.shape[0]
        s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = do @ v.T
    delta = (p * dp).sum(axis=1, keepdims=True)
    ds = np.abs(p * (dp - delta))
    e = np.abs((do * (o_dev - p @ v)).sum(axis=1, keepdims=True))  # |dO_i . (O_gpu,i - O_i)|
    pe = p * e
    mags = (abs(sc) * (ds @ np.abs(k)), abs(sc) * (ds.T @ np.abs(q)), p.T @ np.abs(do))
    props = (abs(sc) * (pe @ np.abs(k)), abs(sc) * (pe.T @ np.abs(q)), np.zeros_like(v))
    return mags, props


@pytest.mark.parametrize("N", [1, 31, 64, 100, 255, 257, 600])
@pytest.mark.parametrize("D", [32, 64, 96, 128, 160, 192, 224, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged(N, D, dtype, causal):
    check_bwd(1, 2, N, D, dtype, causal, seed=700 + N + D)


@pytest.mark.parametrize("N", [1, 31, 64, 100, 255, 257, 600])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_f32_ragged(N, D, causal):
    """fp32 inputs (fp32 matrix instructions throughout), ragged N."""
    check_bwd(1, 2, N, D, "f32", causal, seed=3200 + 17 * N + D)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_f32_several_blocks(D, causal):
    """fp32 over several 128-row query and key blocks with a ragged tail."""
    check_bwd(2, 2, 700, D, "f32", causal, seed=3900 + D)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.3])
def test_bwd_f32_scales(scale):
    """fp32 with a zero, a negative and a large scale."""
    check_bwd(1, 2, 300, 64, "f32", True, seed=4100, scale=scale)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_d96_several_blocks(causal):
    """D = 96 over several query and key blocks with a ragged tail (N = 1100)."""
    check_bwd(1, 3, 1100, 96, "bf16", causal, seed=796)


@pytest.mark.parametrize("D", [192, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_wide_heads_several_blocks(D, causal):
    """D = 192 and 256 (dQ in 128-row blocks; at 256 dV and dK from separate
    launches) over several query and key blocks with a ragged tail (N = 700)."""
    check_bwd(1, 2, 700, D, "bf16", causal, seed=1920 + D)


@pytest.mark.parametrize("D,causal", [(192, False), (256, False), (256, True)])
def test_bwd_wide_heads_full_size_slice(D, causal):
    """B4 H8 N4096 at D = 192 and 256, the shapes and launches bench.py times:
    one seeded (b, h) slice, every row."""
    slices = fi.sample_slices(4, 8, 1, seed=41 + D + int(causal))
    check_bwd(4, 8, 4096, D, "bf16", causal, seed=1004, slices=slices)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_f32_headline_slice(causal):
    """fp32 at the headline shape (B4 H16 N4096 D128), one seeded slice, every row."""
    slices = fi.sample_slices(4, 16, 1, seed=43 + int(causal))
    check_bwd(4, 16, 4096, 128, "f32", causal, seed=1004, slices=slices)


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


def test_bwd_f32_deterministic_and_binding():
    """fp32: two calls agree bit for bit, and the binding's bwd matches the C ABI call."""
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    q, k, v = fi.make_qkv(1, 2, 400, 64, "f32", seed=12)
    do, _, _ = fi.make_qkv(1, 2, 400, 64, "f32", seed=13)
    g1 = run_bwd(q, k, v, do, "f32", 0.125, True)
    g2 = run_bwd(q, k, v, do, "f32", 0.125, True)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    dq_, dk_, dv_, do_ = (_to_device(x, "f32") for x in (q, k, v, do))
    o, lse = fa.fwd(dq_, dk_, dv_, scale=0.125, causal=True)
    g3 = fa.bwd(dq_, dk_, dv_, o, lse, do_, scale=0.125, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g3):
        assert torch.equal(a, b)
