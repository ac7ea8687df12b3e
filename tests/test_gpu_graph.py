"""GPU tests of the library's calls under HIP graph capture (torch.cuda.CUDAGraph).

fa_fwd, fa_fwd_split_static, fa_fwd_varlen and fa_bwd are each captured once
(after one eager call, which sets up the library's per-device state) and the
graph is then replayed several times.  Before every replay, ordinary eager work
on the same stream writes fresh inputs into the captured buffers and poisons
the outputs with NaN, followed by a synchronisation; after it, every output of
the replay must equal, bit for bit, an eager call on the same inputs (the
kernels are deterministic).  The calls allocate nothing and record no memset,
so the graph holds their kernels only.  Every call goes through the C ABI.
"""
import math

import numpy as np
import pytest

import fa_inputs as fi

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dev(x, dtype):
    torch = _torch()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _code(dtype):
    import attention_fa_fwd_02_amd as fa
    return {"f32": fa.FA_DTYPE_F32, "bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16}[dtype]


def _bits(t):
    torch = _torch()
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def _same(a, b):
    torch = _torch()
    return bool(torch.equal(_bits(a), _bits(b)))


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _replay_and_check(graph, refill, outputs, eager):
    """refill(rep) writes fresh inputs (eager); eager() returns the outputs of an
    eager call on them, in the order of `outputs`."""
    torch = _torch()
    for rep in range(REPLAYS):
        refill(rep)
        for t in outputs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = eager()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outputs, ref)):
            assert bool(torch.isfinite(got).all()), "replay %d output %d not fully written" % (rep, i)
            assert _same(got, want), "replay %d output %d differs from the eager call" % (rep, i)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64), ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_graph_fwd(dtype, D, causal):
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    B, H, N = 2, 3, 1000
    scale = 1.0 / math.sqrt(D)
    q, k, v = (_dev(x, dtype) for x in fi.make_qkv(B, H, N, D, dtype, 7100))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    print("graph fa_fwd B%d H%d N%d D%d %s causal=%d" % (B, H, N, D, dtype, causal), flush=True)

    def call(o_, lse_):
        return fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_.data_ptr(), lse_.data_ptr(),
                         B, H, N, D, scale, int(causal), _code(dtype), _stream())

    assert call(o, lse) == fa.FA_OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = call(o, lse)
    assert st == fa.FA_OK, fa.fa_status_string(st)

    def refill(rep):
        for dst, src in zip((q, k, v), fi.make_qkv(B, H, N, D, dtype, 7101 + rep)):
            dst.copy_(_dev(src, dtype))

    def eager():
        o_e, l_e = torch.empty_like(o), torch.empty_like(lse)
        assert call(o_e, l_e) == fa.FA_OK
        return o_e, l_e

    _replay_and_check(g, refill, (o, lse), eager)


@pytest.mark.parametrize("causal", [False, True])
def test_graph_split_static(causal):
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    B, H, N, D, dtype, n_splits = 1, 2, 2000, 128, "bf16", 4
    scale = 1.0 / math.sqrt(D)
    q, k, v = (_dev(x, dtype) for x in fi.make_qkv(B, H, N, D, dtype, 7200))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    print("graph fa_fwd_split_static B%d H%d N%d D%d splits=%d causal=%d" % (B, H, N, D, n_splits, causal),
          flush=True)

    def call(o_, lse_):
        return fa.fa_fwd_split_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_.data_ptr(), lse_.data_ptr(),
                                      B, H, N, D, scale, int(causal), _code(dtype), n_splits, _stream())

    assert call(o, lse) == fa.FA_OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = call(o, lse)
    assert st == fa.FA_OK, fa.fa_status_string(st)

    def refill(rep):
        for dst, src in zip((q, k, v), fi.make_qkv(B, H, N, D, dtype, 7201 + rep)):
            dst.copy_(_dev(src, dtype))

    def eager():
        o_e, l_e = torch.empty_like(o), torch.empty_like(lse)
        assert call(o_e, l_e) == fa.FA_OK
        return o_e, l_e

    _replay_and_check(g, refill, (o, lse), eager)


@pytest.mark.parametrize("causal", [False, True])
def test_graph_varlen(causal):
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    H, D, dtype = 2, 128, "bf16"
    lens_q = np.array([1, 300, 77, 513, 128], dtype=np.int64)
    lens_k = np.array([5, 300, 200, 513, 64], dtype=np.int64)
    cq, ck = fi.cu_seqlens(lens_q), fi.cu_seqlens(lens_k)
    total_q, total_k, n_seqs, max_q = int(cq[-1]), int(ck[-1]), len(lens_q), int(lens_q.max())
    scale = 1.0 / math.sqrt(D)
    q, k, v = (_dev(x, dtype) for x in fi.make_packed(H, total_q, total_k, D, dtype, 7300))
    dcq = torch.from_numpy(cq).to("cuda")
    dck = torch.from_numpy(ck).to("cuda")
    o = torch.empty_like(q)
    lse = torch.empty((H, total_q), dtype=torch.float32, device="cuda")
    print("graph fa_fwd_varlen seqs=%d H%d total_q=%d total_k=%d D%d causal=%d"
          % (n_seqs, H, total_q, total_k, D, causal), flush=True)

    def call(o_, lse_):
        return fa.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_.data_ptr(), lse_.data_ptr(),
                                dcq.data_ptr(), dck.data_ptr(), n_seqs, H, total_q, total_k, max_q, D, scale,
                                int(causal), _code(dtype), _stream())

    assert call(o, lse) == fa.FA_OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = call(o, lse)
    assert st == fa.FA_OK, fa.fa_status_string(st)

    def refill(rep):
        for dst, src in zip((q, k, v), fi.make_packed(H, total_q, total_k, D, dtype, 7301 + rep)):
            dst.copy_(_dev(src, dtype))

    def eager():
        o_e, l_e = torch.empty_like(o), torch.empty_like(lse)
        assert call(o_e, l_e) == fa.FA_OK
        return o_e, l_e

    # a causal row whose query sees no key (cross lengths) has lse = -inf: compare those as bits
    torch_isfinite = torch.isfinite
    for rep in range(REPLAYS):
        refill(rep)
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e, l_e = eager()
        torch.cuda.synchronize()
        assert bool(torch_isfinite(o).all()), "replay %d O not fully written" % rep
        assert not bool(torch.isnan(lse).any()), "replay %d lse not fully written" % rep
        assert _same(o, o_e), "replay %d O differs from the eager call" % rep
        assert _same(lse, l_e), "replay %d lse differs from the eager call" % rep


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 256), ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_graph_bwd(dtype, D, causal):
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    B, H, N = 1, 2, 700
    scale = 1.0 / math.sqrt(D)
    q, k, v = (_dev(x, dtype) for x in fi.make_qkv(B, H, N, D, dtype, 7400))
    do = _dev(fi.make_qkv(B, H, N, D, dtype, 7400 + 7919)[0], dtype)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsb = fa.fa_bwd_workspace_bytes(B, H, N, D)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    print("graph fa_bwd B%d H%d N%d D%d %s causal=%d" % (B, H, N, D, dtype, causal), flush=True)

    def forward():
        assert fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, D,
                         scale, int(causal), _code(dtype), _stream()) == fa.FA_OK

    def call(dq_, dk_, dv_):
        return fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                         dq_.data_ptr(), dk_.data_ptr(), dv_.data_ptr(), B, H, N, D, scale, int(causal),
                         _code(dtype), ws.data_ptr(), wsb, _stream())

    forward()
    assert call(dq, dk, dv) == fa.FA_OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = call(dq, dk, dv)
    assert st == fa.FA_OK, fa.fa_status_string(st)

    def refill(rep):
        seed = 7401 + rep
        for dst, src in zip((q, k, v), fi.make_qkv(B, H, N, D, dtype, seed)):
            dst.copy_(_dev(src, dtype))
        do.copy_(_dev(fi.make_qkv(B, H, N, D, dtype, seed + 7919)[0], dtype))
        forward()  # O and lse of the new inputs, eagerly

    def eager():
        outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        assert call(*outs) == fa.FA_OK
        return outs

    _replay_and_check(g, refill, (dq, dk, dv), eager)
