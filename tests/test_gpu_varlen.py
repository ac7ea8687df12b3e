"""GPU parity of packed variable-length attention (fa_fwd_varlen, through the C ABI).

Head-major packed Q [H, total_q, D], K/V [H, total_k, D] with int32
cu_seqlens on the device; each sequence is checked against the fp64 oracle
for packed sequences (bottom-right causal), every row for small batches and
seeded row samples for the full length-mix workload.  Rows that see no key
must come back as O = 0 and lse = -inf.  Outputs start poisoned (NaN) and are
followed by guard bands.  Tolerances are those of fa_fwd (fp32 1e-5; bf16 /
fp16 1e-2 on O and 1e-3 on lse, plus half an output ulp where |O| >= 4).
"""
import math

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.test_gpu_parity import TOL, GUARD, _host_widen, _tdtype, _to_device, _torch, half_ulp

pytestmark = pytest.mark.gpu


def run_varlen(q, k, v, cu_q, cu_k, max_q, dtype, scale, causal):
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    H, total_q, D = q.shape
    total_k = k.shape[1]
    n_o, n_l = H * total_q * D, H * total_q
    td = _tdtype(dtype)
    o_buf = torch.full((n_o + GUARD,), float("nan"), dtype=td, device="cuda")
    l_buf = torch.full((n_l + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    o_buf[n_o:] = 7.0
    l_buf[n_l:] = -3.0
    dq, dk, dv = (_to_device(x, dtype) for x in (q, k, v))
    dcq = torch.from_numpy(np.asarray(cu_q, dtype=np.int32)).to("cuda")
    dck = torch.from_numpy(np.asarray(cu_k, dtype=np.int32)).to("cuda")
    code = {"f32": fa.FA_DTYPE_F32, "bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16}[dtype]
    n_seqs = len(cu_q) - 1
    print("fa_fwd_varlen seqs=%d H%d total_q=%d total_k=%d D%d %s causal=%d" %
          (n_seqs, H, total_q, total_k, D, dtype, causal), flush=True)
    st = fa.fa_fwd_varlen(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), o_buf.data_ptr(), l_buf.data_ptr(),
                          dcq.data_ptr(), dck.data_ptr(), n_seqs, H, total_q, total_k, max_q, D, float(scale),
                          int(causal), code, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    assert torch.all(o_buf[n_o:] == 7.0), "O guard band overwritten"
    assert torch.all(l_buf[n_l:] == -3.0), "lse guard band overwritten"
    o = o_buf[:n_o].view(H, total_q, D)
    lse = l_buf[:n_l].view(H, total_q)
    assert bool(torch.isfinite(o).all()), "O has unwritten or non-finite elements"
    assert not bool(torch.isnan(lse).any()), "lse has unwritten elements"
    return o, lse


def check_varlen(lens_q, lens_k, H, D, dtype, causal, seed, n_rows=None, scale=None):
    cu_q, cu_k = fi.cu_seqlens(lens_q), fi.cu_seqlens(lens_k)
    total_q, total_k = int(cu_q[-1]), int(cu_k[-1])
    q, k, v = fi.make_packed(H, total_q, total_k, D, dtype, seed)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    o, lse = run_varlen(q, k, v, cu_q, cu_k, max(1, int(max(lens_q))), dtype, scale, causal)
    tol_o, tol_l = TOL[dtype]
    rows_of = None if n_rows is None else (lambda b: fi.sample_rows(int(lens_q[b]), n_rows, seed=seed + b))
    ref = oracle.attention_varlen(oracle.widen(q, dtype), oracle.widen(k, dtype), oracle.widen(v, dtype),
                                  cu_q, cu_k, oracle.gpu_scale(scale), causal, rows_of=rows_of)
    worst_o = worst_l = 0.0
    n_empty = 0
    for b, rows, o_ref, l_ref in ref:
        if rows.size == 0:
            continue
        idx = int(cu_q[b]) + rows
        o_got = _host_widen(o[:, idx], dtype)
        l_got = lse[:, idx].cpu().numpy().astype(np.float64)
        empty = l_ref == -np.inf
        n_empty += int(empty.sum())
        assert np.array_equal(l_got == -np.inf, empty), "sequence %d: rows without keys differ" % b
        assert np.all(o_got[empty] == 0.0), "sequence %d: a row without keys has O != 0" % b
        d_o = np.abs(o_got - o_ref)
        tol = tol_o + np.where(np.abs(o_ref) >= 4.0, half_ulp(o_ref, dtype), 0.0)
        assert (d_o <= tol).all(), (b, float(d_o.max()))
        if (~empty).any():
            d_l = float(np.abs(l_got[~empty] - l_ref[~empty]).max())
            assert d_l <= tol_l, (b, d_l)
            worst_l = max(worst_l, d_l)
        worst_o = max(worst_o, float(d_o.max()))
    print("  max|dO|=%.3g max|dlse|=%.3g  (%d rows without keys)" % (worst_o, worst_l, n_empty), flush=True)
    return q, k, v, o, lse


# self-attention mixes (n_q = n_k per sequence): empty, single-row, ragged and
# multi-block sequences
MIX_SELF = [1, 0, 255, 257, 600, 31, 1000]
# cross mixes: n_q < n_k, n_q > n_k (causal rows without keys), n_k = 0, n_q = 0
MIX_Q = [5, 300, 0, 700, 40, 129]
MIX_K = [900, 100, 50, 700, 0, 1]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_self(D, dtype, causal):
    check_varlen(MIX_SELF, MIX_SELF, 3, D, dtype, causal, seed=500 + D)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_cross(D, dtype, causal):
    check_varlen(MIX_Q, MIX_K, 2, D, dtype, causal, seed=600 + D)


@pytest.mark.parametrize("D", [32, 96, 160, 192, 224, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_head_dims(D, causal):
    check_varlen(MIX_Q, MIX_K, 2, D, "bf16", causal, seed=650 + D)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_workload_sampled(causal):
    """The 16-sequence length mix (128..4096 keys, H16 D128 bf16): 48 rows per sequence."""
    w = fi.VARLEN_WORKLOAD
    lens = fi.make_seqlens(w["n_seqs"], w["lo"], w["hi"], w["seed"])
    check_varlen(lens, lens, w["H"], w["D"], w["dtype"], causal, w["seed"], n_rows=48)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_match_dense(dtype, causal):
    """Equal square sequences, packed head-major, give the same bits as fa_fwd on
    the [B, H, N, D] layout of the same data (same arithmetic, same order).  The
    grid is large enough that fa_fwd takes whole key tiles per wave (no key
    groups, whose partials are combined in another order)."""
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    B, H, N, D = 4, 64, 1000, 64
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    name = fa.fa_fwd_kernel_name(B, H, N, D, int(causal), 1 if dtype == "bf16" else 0, n_cus)
    assert name.endswith(", 1>") or dtype == "f32", name
    q, k, v = fi.make_qkv(B, H, N, D, dtype, seed=77)
    pack = lambda x: np.ascontiguousarray(x.transpose(1, 0, 2, 3).reshape(H, B * N, D))
    cu = fi.cu_seqlens([N] * B)
    o, lse = run_varlen(pack(q), pack(k), pack(v), cu, cu, N, dtype, 0.125, causal)
    dq, dk, dv = (_to_device(x, dtype) for x in (q, k, v))
    od, ld = fa.fwd(dq, dk, dv, scale=0.125, causal=causal)
    torch.cuda.synchronize()
    od_p = od.permute(1, 0, 2, 3).reshape(H, B * N, D)
    ld_p = ld.permute(1, 0, 2).reshape(H, B * N)
    if dtype == "bf16":
        assert torch.equal(o.view(torch.int16), od_p.contiguous().view(torch.int16))
    else:
        assert torch.equal(o, od_p)
    assert torch.equal(lse, ld_p)


def test_varlen_binding():
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    lens_q, lens_k = [3, 400, 77], [500, 400, 1]
    cu_q, cu_k = fi.cu_seqlens(lens_q), fi.cu_seqlens(lens_k)
    q, k, v = fi.make_packed(2, int(cu_q[-1]), int(cu_k[-1]), 128, "bf16", seed=78)
    o1, l1 = run_varlen(q, k, v, cu_q, cu_k, 400, "bf16", 1 / math.sqrt(128), True)
    dq, dk, dv = (_to_device(x, "bf16") for x in (q, k, v))
    dcq, dck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = fa.fwd_varlen(dq, dk, dv, dcq, dck, 400, causal=True)
    s.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
