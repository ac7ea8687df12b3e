"""GPU parity of the key-split path and the lse merge (through the C ABI).

fa_fwd_split computes n_splits key-range partials into the caller's
workspace and merges them on the device.  Checked against the fp64 oracle
on the same seeded inputs:
  * the merged O and lse, every row, with the tolerances of fa_fwd
    (fp32 1e-5; bf16 / fp16 1e-2 on O, 1e-3 on lse);
  * every split's partial (normalised O over the split's key range and its
    lse) against the oracle restricted to that range, read back from the
    workspace; rows that see no key of a split must have lse = -inf;
  * fa_lse_merge on its own against the oracle's merge, with empty parts
    whose O is NaN (it must not be read) and rows whose parts are all empty.
Outputs and the workspace start poisoned (NaN) and are followed by guard
bands that must stay untouched.
"""
import math

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.test_gpu_parity import TOL, GUARD, _host_widen, _tdtype, _to_device, _torch, half_ulp

pytestmark = pytest.mark.gpu

N_CUS = 256  # MI355X compute units, for the library's split-count choice


def key_ranges(N, n_splits):
    """[lo, hi) of each split as the C header defines it: whole 128-key tiles,
    ceil(tiles / n_splits) tiles per split."""
    tiles = (N + 127) // 128
    keys = 128 * ((tiles + n_splits - 1) // n_splits)
    return [(min(N, s * keys), min(N, (s + 1) * keys)) for s in range(n_splits)]


def run_split(q, k, v, dtype, scale, causal, n_splits):
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    B, H, N, D = q.shape
    n_o, n_l = B * H * N * D, B * H * N
    td = _tdtype(dtype)
    o_buf = torch.full((n_o + GUARD,), float("nan"), dtype=td, device="cuda")
    l_buf = torch.full((n_l + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    o_buf[n_o:] = 7.0
    l_buf[n_l:] = -3.0
    ws_bytes = fa.fa_fwd_split_workspace_bytes(B, H, N, D, n_splits)
    assert ws_bytes == n_splits * n_l * (D + 1) * 4
    ws = torch.full((ws_bytes // 4 + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    ws[ws_bytes // 4:] = 5.0
    dq, dk, dv = (_to_device(x, dtype) for x in (q, k, v))
    code = {"f32": fa.FA_DTYPE_F32, "bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16}[dtype]
    print("fa_fwd_split B%d H%d N%d D%d %s causal=%d splits=%d" % (B, H, N, D, dtype, causal, n_splits),
          flush=True)
    st = fa.fa_fwd_split(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), o_buf.data_ptr(), l_buf.data_ptr(),
                         B, H, N, D, float(scale), int(causal), code, n_splits, ws.data_ptr(), ws_bytes,
                         torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    assert torch.all(o_buf[n_o:] == 7.0), "O guard band overwritten"
    assert torch.all(l_buf[n_l:] == -3.0), "lse guard band overwritten"
    assert torch.all(ws[ws_bytes // 4:] == 5.0), "workspace guard band overwritten"
    o = o_buf[:n_o].view(B, H, N, D)
    lse = l_buf[:n_l].view(B, H, N)
    assert bool(torch.isfinite(o).all()), "O has unwritten or non-finite elements"
    assert bool(torch.isfinite(lse).all()), "lse has unwritten or non-finite elements"
    part_o = ws[:n_splits * n_o].view(n_splits, B, H, N, D)
    part_lse = ws[n_splits * n_o:n_splits * n_o + n_splits * n_l].view(n_splits, B, H, N)
    return o, lse, part_o, part_lse


def check_split(B, H, N, D, dtype, causal, n_splits, seed, slices=None, n_rows=None, partials=True):
    q, k, v = fi.make_qkv(B, H, N, D, dtype, seed)
    scale = 1.0 / math.sqrt(D)
    sc = oracle.gpu_scale(scale)
    o, lse, part_o, part_lse = run_split(q, k, v, dtype, scale, causal, n_splits)
    tol_o, tol_l = TOL[dtype]
    ranges = key_ranges(N, n_splits)
    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    worst = [0.0, 0.0, 0.0, 0.0]
    for (b, h) in slices:
        rows = (np.arange(N, dtype=np.int64) if n_rows is None
                else fi.sample_rows(N, n_rows, seed=seed + 1000 * b + h))
        qw = oracle.widen(q[b, h][rows], dtype)
        kw = oracle.widen(k[b, h], dtype)
        vw = oracle.widen(v[b, h], dtype)
        o_ref, l_ref = oracle.attention_rows(qw, kw, vw, rows, sc, causal)
        o_got = _host_widen(o[b, h][rows], dtype)
        l_got = lse[b, h][rows].cpu().numpy().astype(np.float64)
        d_o = np.abs(o_got - o_ref)
        tol = tol_o + np.where(np.abs(o_ref) >= 4.0, half_ulp(o_ref, dtype), 0.0)
        assert (d_o <= tol).all(), float(d_o.max())
        assert np.abs(l_got - l_ref).max() <= tol_l
        worst[0] = max(worst[0], float(d_o.max()))
        worst[1] = max(worst[1], float(np.abs(l_got - l_ref).max()))
        if not partials:
            continue
        for s, (lo, hi) in enumerate(ranges):
            po_ref, pl_ref = oracle.attention_rows(qw, kw, vw, rows, sc, causal, key_range=(lo, hi))
            pl_got = part_lse[s, b, h][rows].cpu().numpy().astype(np.float64)
            empty = pl_ref == -np.inf
            assert np.array_equal(pl_got == -np.inf, empty), "split %d: empty rows differ" % s
            if empty.all():
                continue
            po_got = part_o[s, b, h][rows].cpu().numpy().astype(np.float64)
            dpo = np.abs(po_got[~empty] - po_ref[~empty])
            dpl = np.abs(pl_got[~empty] - pl_ref[~empty])
            assert dpo.max() <= tol_o, (s, float(dpo.max()))
            assert dpl.max() <= tol_l, (s, float(dpl.max()))
            worst[2] = max(worst[2], float(dpo.max()))
            worst[3] = max(worst[3], float(dpl.max()))
    print("  merged max|dO|=%.3g max|dlse|=%.3g; partials max|dO|=%.3g max|dlse|=%.3g" % tuple(worst),
          flush=True)
    return q, k, v, o, lse


@pytest.mark.parametrize("N,n_splits", [(1000, 3), (1, 3), (129, 2), (300, 64)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_split_parity(N, n_splits, D, dtype, causal):
    check_split(2, 3, N, D, dtype, causal, n_splits, seed=300 + N + D)


@pytest.mark.parametrize("D", [32, 96, 160, 192, 224, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_split_head_dims(D, causal):
    check_split(2, 3, 1000, D, "bf16", causal, 3, seed=350 + D)


@pytest.mark.parametrize("causal", [False, True])
def test_split_small_workload(causal):
    """The small bf16 workload in four splits (64 workgroups x 4 fill 256 CUs; the
    library's own choice there is 1, its 8 key tiles being too few to split),
    also compared with the unsplit fa_fwd on the same inputs."""
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    w = fi.WORKLOADS["small_bf16"]
    assert fa.fa_fwd_split_choose(w["B"], w["H"], w["N"], w["D"], int(causal), N_CUS) == 1
    q, k, v, o, lse = check_split(w["B"], w["H"], w["N"], w["D"], "bf16", causal, 4, w["seed"])
    dq, dk, dv = (_to_device(x, "bf16") for x in (q, k, v))
    o1, l1 = fa.fwd(dq, dk, dv, causal=causal)
    torch.cuda.synchronize()
    assert float((o1.float() - o.float()).abs().max()) <= 2e-2
    assert float((l1 - lse).abs().max()) <= 2e-3


@pytest.mark.parametrize("causal", [False, True])
def test_split_long_sampled(causal):
    """A long sequence on few slices (the case splits are for): sampled rows."""
    import attention_fa_fwd_02_amd as fa
    S = fa.fa_fwd_split_choose(1, 2, 8192, 128, int(causal), N_CUS)
    assert S == 4
    check_split(1, 2, 8192, 128, "bf16", causal, S, seed=41, n_rows=96)


def test_split_deterministic_and_binding():
    """Two calls give identical bits; the convenience binding matches the raw call."""
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    q, k, v = fi.make_qkv(1, 3, 900, 128, "bf16", seed=42)
    o1, l1, _, _ = run_split(q, k, v, "bf16", 1 / math.sqrt(128), True, 5)
    o2, l2, _, _ = run_split(q, k, v, "bf16", 1 / math.sqrt(128), True, 5)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    dq, dk, dv = (_to_device(x, "bf16") for x in (q, k, v))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o3, l3, ws = fa.fwd_split(dq, dk, dv, causal=True, n_splits=5)
    s.synchronize()
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)
    assert ws.numel() >= fa.fa_fwd_split_workspace_bytes(1, 3, 900, 128, 5)


# ------------------------------------------------------------------ merge

def _merge_inputs(P, rows, D, seed):
    rng = np.random.default_rng(seed)
    po = rng.uniform(-2.0, 2.0, size=(P, rows, D)).astype(np.float32)
    pl = (rng.standard_normal((P, rows)) * 4.0).astype(np.float32)
    pl[rng.random((P, rows)) < 0.25] = -np.inf
    pl[:, :3] = -np.inf           # rows whose parts are all empty
    pl[0, 3] = 80.0               # one part far above the others
    po[pl == -np.inf] = np.nan    # an empty part's O must not be read
    return po, pl


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [8, 64, 96, 128, 192, 512])
@pytest.mark.parametrize("P", [1, 3, 7])
def test_merge_parity(out, D, P):
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    rows = 1001
    po, pl = _merge_inputs(P, rows, D, seed=50 + P + D)
    d_po = torch.from_numpy(po).to("cuda")
    d_pl = torch.from_numpy(pl).to("cuda")
    td = _tdtype(out)
    o_buf = torch.full((rows * D + GUARD,), float("nan"), dtype=td, device="cuda")
    l_buf = torch.full((rows + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    o_buf[rows * D:] = 7.0
    l_buf[rows:] = -3.0
    code = {"f32": fa.FA_DTYPE_F32, "bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16}[out]
    print("fa_lse_merge P%d rows%d D%d -> %s" % (P, rows, D, out), flush=True)
    st = fa.fa_lse_merge(d_po.data_ptr(), d_pl.data_ptr(), P, rows, D, o_buf.data_ptr(), l_buf.data_ptr(),
                         code, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    assert torch.all(o_buf[rows * D:] == 7.0) and torch.all(l_buf[rows:] == -3.0), "guard band overwritten"
    o_ref, l_ref = oracle.lse_merge(po.astype(np.float64), pl.astype(np.float64))
    o_got = _host_widen(o_buf[:rows * D].view(rows, D), out)
    l_got = l_buf[:rows].cpu().numpy().astype(np.float64)
    assert np.isfinite(o_got).all()
    assert np.array_equal(l_got == -np.inf, l_ref == -np.inf)
    fin = np.isfinite(l_ref)
    d_o = np.abs(o_got - o_ref).max()
    d_l = np.abs(l_got[fin] - l_ref[fin]).max()
    tol_o = 1e-5 if out == "f32" else float(half_ulp(np.array([2.0]), out)[0]) + 1e-5
    print("  max|dO|=%.3g max|dlse|=%.3g (tol O %.3g, lse 1e-5)" % (d_o, d_l, tol_o), flush=True)
    assert d_o <= tol_o
    assert d_l <= 1e-5 * max(1.0, float(np.abs(l_ref[fin]).max()))


def test_merge_binding_shapes():
    """The convenience binding: part_o [P, B, H, N, D] -> O [B, H, N, D]."""
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    po, pl = _merge_inputs(2, 2 * 3 * 50, 64, seed=60)
    d_po = torch.from_numpy(po).to("cuda").view(2, 2, 3, 50, 64)
    d_pl = torch.from_numpy(pl).to("cuda").view(2, 2, 3, 50)
    o, l = fa.lse_merge(d_po, d_pl, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 50, 64) and o.dtype == torch.bfloat16 and l.shape == (2, 3, 50)
    o_ref, l_ref = oracle.lse_merge(po.astype(np.float64), pl.astype(np.float64))
    assert np.abs(o.float().cpu().numpy().reshape(-1, 64) - o_ref).max() <= 1e-2
