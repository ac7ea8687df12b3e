"""GPU test of fa_fwd_split_static (the key-split forward pass with its partials
in the library's static device array) against fa_fwd_split with a caller
workspace: the same kernels, so the outputs must agree bit for bit, on two
calls in a row, the second one smaller than the first (the array keeps the
first call's partials, which the second must not pick up)."""
import math

import numpy as np
import pytest

import fa_inputs as fi

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _call(entry, q, k, v, B, H, N, D, dtype, causal, n_splits):
    import attention_fa_fwd_02_amd as fa
    torch = _torch()
    code = {"bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16, "f32": fa.FA_DTYPE_F32}[dtype]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    scale = 1.0 / math.sqrt(D)
    print("%s B%d H%d N%d D%d %s causal=%d splits=%d" % (entry, B, H, N, D, dtype, causal, n_splits), flush=True)
    if entry == "static":
        st = fa.fa_fwd_split_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    B, H, N, D, scale, int(causal), code, n_splits, s)
    else:
        wsb = fa.fa_fwd_split_workspace_bytes(B, H, N, D, n_splits)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        st = fa.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             B, H, N, D, scale, int(causal), code, n_splits, ws.data_ptr(), wsb, s)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return o, lse


def _inputs(B, H, N, D, dtype, seed):
    torch = _torch()
    q, k, v = fi.make_qkv(B, H, N, D, dtype, seed)
    if dtype == "bf16":
        up = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda")
    else:
        up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    return up(q), up(k), up(v)


@pytest.mark.parametrize("causal", [False, True])
def test_static_scratch_matches_workspace_path(causal):
    torch = _torch()
    # a large call, then a smaller one: (B, H, N, D, dtype, n_splits)
    for (B, H, N, D, dtype, n_splits) in ((1, 2, 4096, 128, "bf16", 4), (2, 1, 300, 64, "bf16", 3),
                                          (1, 1, 1000, 64, "f32", 2)):
        q, k, v = _inputs(B, H, N, D, dtype, seed=4100 + N)
        o_s, l_s = _call("static", q, k, v, B, H, N, D, dtype, causal, n_splits)
        o_w, l_w = _call("workspace", q, k, v, B, H, N, D, dtype, causal, n_splits)
        assert bool(torch.isfinite(o_s).all()) and bool(torch.isfinite(l_s).all())
        assert torch.equal(o_s.view(torch.int16) if dtype == "bf16" else o_s,
                           o_w.view(torch.int16) if dtype == "bf16" else o_w)
        assert torch.equal(l_s, l_w)
