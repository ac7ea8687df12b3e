"""GPU parity of fa_fwd's key-group launches (16-bit kernel for D <= 128, fp32
kernel for D = 64).

fa_fwd picks 1, 2 or 4 key groups from the grid size and the device's
compute-unit count (fewer workgroups than compute units: more groups, smaller
query blocks).  The other parity tests mostly use small grids, which take 4
groups; the cases here pin each group count, with ragged N in both modes,
and check the choice through fa_fwd_kernel_name."""
import math

import numpy as np
import pytest

import fa_inputs as fi
from tests.test_gpu_parity import _torch, check_case

pytestmark = pytest.mark.gpu


def _n_cus():
    torch = _torch()
    return torch.cuda.get_device_properties(0).multi_processor_count


def _groups(B, H, N, D, dtype, causal):
    import attention_fa_fwd_02_amd as fa
    code = {"bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16, "f32": fa.FA_DTYPE_F32}[dtype]
    name = fa.fa_fwd_kernel_name(B, H, N, D, int(causal), code, _n_cus())
    print("  kernel:", name, flush=True)
    return int(name.rstrip(">").split(",")[-1])


# (B, H, N): grids of B*H*ceil(N/256) workgroups against 256 compute units
KG1 = [(16, 32, 1000), (16, 32, 2000)]   # 2048 / 4096 workgroups: whole rounds, no split
KG2 = [(2, 50, 200), (2, 40, 300), (1, 100, 255)]
KG4 = [(2, 8, 1024), (1, 3, 100), (2, 2, 129), (1, 1, 1000)]


# (dtype, D) pairs: every 16-bit head dim of the kernel; fp32 at D = 64 (key
# groups) and, with whole tiles only, D = 128
DT_KG1 = [("bf16", 64), ("bf16", 96), ("bf16", 128), ("f32", 64), ("f32", 128)]
DT_KG = [(t, d) for t in ("bf16", "f16") for d in (32, 64, 96, 128)] + [("f32", 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,D", DT_KG1)
@pytest.mark.parametrize("shape", KG1)
def test_one_group_ragged(shape, dtype, D, causal):
    B, H, N = shape
    if _n_cus() == 256:
        assert _groups(B, H, N, D, dtype, causal) == 1
    slices = fi.sample_slices(B, H, 6, seed=31)
    check_case(B, H, N, D, dtype, causal, seed=300 + N + D, slices=slices)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,D", DT_KG)
@pytest.mark.parametrize("shape", KG2)
def test_two_groups(shape, dtype, D, causal):
    B, H, N = shape
    if _n_cus() == 256:
        assert _groups(B, H, N, D, dtype, causal) == 2
    slices = fi.sample_slices(B, H, 12, seed=32)
    check_case(B, H, N, D, dtype, causal, seed=400 + N + D, slices=slices)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,D", DT_KG)
@pytest.mark.parametrize("shape", KG4)
def test_four_groups(shape, dtype, D, causal):
    B, H, N = shape
    if _n_cus() == 256:
        assert _groups(B, H, N, D, dtype, causal) == 4
    check_case(B, H, N, D, dtype, causal, seed=500 + N + D)


def test_key_groups_deterministic():
    """Two calls give bitwise the same output in every group count."""
    from tests.test_gpu_parity import run_fa
    torch = _torch()
    for (B, H, N) in (KG1[0], KG2[0], KG4[0]):
        q, k, v = fi.make_qkv(B, H, N, 128, "bf16", seed=33)
        o1, l1 = run_fa(q, k, v, "bf16", 1 / math.sqrt(128), True)
        o2, l2 = run_fa(q, k, v, "bf16", 1 / math.sqrt(128), True)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
        q, k, v = fi.make_qkv(B, H, N, 64, "f32", seed=34)
        o1, l1 = run_fa(q, k, v, "f32", 0.125, True)
        o2, l2 = run_fa(q, k, v, "f32", 0.125, True)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
