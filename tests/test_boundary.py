"""CPU tests of the C-ABI boundary: the library loads, exports every symbol the
header declares, and every argument error is reported on the host before any
HIP call (no compute calls here)."""
import os
import re

import pytest

import attention_fa_fwd_02_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")



@pytest.fixture(autouse=True)
def _library(libfa):
    """Every test here needs the built library: a missing or broken build fails them."""
    return libfa


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = fa.load_library()
    names = declared_functions()
    assert set(names) == {"fa_fwd", "fa_check_args", "fa_status_string", "fa_abi_version",
                          "fa_fwd_split", "fa_fwd_split_workspace_bytes", "fa_fwd_split_choose",
                          "fa_lse_merge", "fa_fwd_varlen", "fa_check_varlen_args", "fa_bwd",
                          "fa_bwd_workspace_bytes", "fa_check_bwd_args", "fa_fwd_fp8",
                          "fa_fwd_fp8_workspace_bytes", "fa_check_fp8_args", "fa_fwd_kernel_name",
                          "fa_fwd_split_static"}
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_matches_header():
    m = re.search(r"#define FA_ABI_VERSION (\d+)", open(HEADER).read())
    assert fa.fa_abi_version() == int(m.group(1))


def test_status_strings():
    for s in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP):
        assert fa.fa_status_string(s)
    assert fa.fa_status_string(99) == "unknown status"


# fake, well-separated, aligned device addresses: only compared, never dereferenced
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
T = 1 << 40  # address spacing for the large cases: no two tensors overlap
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, N=100, D=64, scale=0.125, causal=0, dtype=1)


def check(arch="gfx950:sramecc+:xnack-", **kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_check_args(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["D"],
                            a["scale"], a["causal"], a["dtype"], arch)


def test_good_arguments_pass():
    assert check() == fa.FA_OK
    assert check(arch=None) == fa.FA_OK
    for dt in (0, 1, 2):
        for D in (64, 128):
            for c in (0, 1):
                assert check(dtype=dt, D=D, causal=c) == fa.FA_OK
    assert check(scale=0.0) == fa.FA_OK
    assert check(scale=-0.5) == fa.FA_OK
    assert check(N=1, B=1, H=1) == fa.FA_OK


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(lse=0),
    dict(B=0), dict(H=-1), dict(N=0), dict(D=0),
    dict(scale=float("nan")), dict(scale=float("inf")), dict(scale=float("-inf")),
    dict(causal=2), dict(causal=-1), dict(dtype=3), dict(dtype=-1),
    dict(q=Q + 8), dict(k=K + 2), dict(v=V + 4), dict(o=O + 1), dict(lse=L + 2),
    dict(o=Q), dict(o=K + 64), dict(o=V - 16), dict(lse=Q + 4), dict(lse=O + 16), dict(o=L - 32),
])
def test_invalid_arguments(kw):
    assert check(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(D=16), dict(D=48), dict(D=80), dict(D=288), dict(D=512), dict(D=96, dtype=0), dict(D=256, dtype=0),
    dict(D=32, dtype=0), dict(D=160, dtype=0),
    dict(N=1 << 30), dict(B=1 << 20, H=1 << 10, N=1 << 7), dict(B=1 << 15, H=1 << 8, N=257),
    # head dims above 192 use 128-row query blocks: 2^16 * 2^7 blocks of 128 rows
    dict(B=1 << 16, H=1 << 0, N=128 * 128, D=256, q=T, k=2 * T, v=3 * T, o=4 * T, lse=5 * T),
])
def test_unsupported(kw):
    assert check(**kw) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", [1, 2])
@pytest.mark.parametrize("D", [32, 64, 96, 128, 160, 192, 224, 256])
def test_head_dims_16bit(D, dtype):
    assert check(D=D, dtype=dtype) == fa.FA_OK


def test_grid_limit_depends_on_query_block():
    """2^22 query blocks of 256 rows pass at D = 128; the same N at D = 256 needs 2^23
    blocks of 128 rows and is refused."""
    big = dict(B=1 << 14, H=1 << 0, N=256 * 256, q=T, k=2 * T, v=3 * T, o=4 * T, lse=5 * T)
    assert check(D=128, **big) == fa.FA_OK
    assert check(D=256, **big) == fa.FA_ERR_UNSUPPORTED


def test_kernel_name():
    """The dispatch's kernel, named as the profiler reports it; "" for sizes fa_fwd rejects."""
    assert fa.fa_fwd_kernel_name(4, 16, 4096, 128, 0, 1, 256) == "fa_fwd_pp_kernel<Bf16, 128, false, 0, 1>"
    assert fa.fa_fwd_kernel_name(4, 8, 4096, 256, 1, 2, 256) == "fa_fwd_mfma_kernel<F16, 256, true, 0>"
    # D = 192: the ping-pong kernel without the causal mask, the one-barrier kernel with it
    assert fa.fa_fwd_kernel_name(4, 8, 4096, 192, 0, 1, 256) == "fa_fwd_pp_kernel<Bf16, 192, false, 0, 1>"
    assert fa.fa_fwd_kernel_name(4, 8, 4096, 192, 1, 1, 256) == "fa_fwd_mfma_kernel<Bf16, 192, true, 0>"
    # D = 160 like 192; D = 32 like 64 (key groups included)
    assert fa.fa_fwd_kernel_name(4, 8, 4096, 160, 0, 2, 256) == "fa_fwd_pp_kernel<F16, 160, false, 0, 1>"
    assert fa.fa_fwd_kernel_name(4, 8, 4096, 160, 1, 1, 256) == "fa_fwd_mfma_kernel<Bf16, 160, true, 0>"
    assert fa.fa_fwd_kernel_name(4, 16, 4096, 32, 1, 1, 256) == "fa_fwd_pp_kernel<Bf16, 32, true, 0, 1>"
    assert fa.fa_fwd_kernel_name(2, 8, 1024, 32, 0, 1, 256) == "fa_fwd_pp_kernel<Bf16, 32, false, 0, 4>"
    # D = 224 like 256: four waves, the one-barrier kernel in every mode
    assert fa.fa_fwd_kernel_name(4, 8, 4096, 224, 0, 1, 256) == "fa_fwd_mfma_kernel<Bf16, 224, false, 0>"
    assert fa.fa_fwd_kernel_name(1, 1, 128, 32, 0, 0, 256) == ""
    assert fa.fa_fwd_kernel_name(1, 1, 128, 64, 0, 0, 256).startswith("fa_fwd_f32_kernel<64, false")
    # small grids take key groups: B2 H8 N1024 is 64 workgroups of 256 rows on 256 CUs
    assert fa.fa_fwd_kernel_name(2, 8, 1024, 64, 1, 1, 256) == "fa_fwd_pp_kernel<Bf16, 64, true, 0, 4>"
    assert fa.fa_fwd_kernel_name(2, 50, 200, 96, 0, 2, 256) == "fa_fwd_pp_kernel<F16, 96, false, 0, 2>"
    assert fa.fa_fwd_kernel_name(1, 1, 128, 48, 0, 1, 256) == ""
    assert fa.fa_fwd_kernel_name(1, 1, 128, 64, 2, 1, 256) == ""
    assert fa.fa_fwd_kernel_name(1, 1, 128, 64, 0, 1, 0) == ""


def test_unsupported_arch():
    assert check(arch="gfx942:sramecc+:xnack-") == fa.FA_ERR_UNSUPPORTED
    assert check(arch="gfx1100") == fa.FA_ERR_UNSUPPORTED


def test_fwd_reports_invalid_args_before_any_hip_call():
    # NULL q: rejected on the host, so this is safe without a GPU
    st = fa.fa_fwd(0, K, V, O, L, 1, 1, 64, 64, 0.125, 0, 1, 0)
    assert st == fa.FA_ERR_INVALID_ARG
    st = fa.fa_fwd(Q, K, V, O, L, 1, 1, 64, 48, 0.125, 0, 1, 0)
    assert st == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("B,H,N", [(1 << 35, 1 << 35, 1), (1 << 31, 1, 1), (1, 1 << 31, 1),
                                    (1 << 30, 1 << 30, 1 << 10), ((1 << 62) + 1, 4, 1)])
def test_size_products_do_not_wrap(B, H, N):
    """B*H (and B*H*N) beyond the limits are refused even where the 64-bit
    product would wrap to a small value (2^35 * 2^35 = 2^70 wraps to 0)."""
    big = dict(q=T, k=2 * T, v=3 * T, o=4 * T, lse=5 * T)
    assert check(B=B, H=H, N=N, **big) == fa.FA_ERR_UNSUPPORTED
    assert bcheck(B=B, H=H, N=N, q=T, k=2 * T, v=3 * T, o=4 * T, do=5 * T, lse=6 * T, dq=7 * T, dk=8 * T,
                  dv=9 * T, ws=10 * T, wsb=1 << 62) == fa.FA_ERR_UNSUPPORTED
    if N < (1 << 24):
        assert f8check(B=B, H=H, N=N, wsb=1 << 62) == fa.FA_ERR_UNSUPPORTED


class _FakeDeviceTensor:
    """Duck-typed stand-in for a device tensor (no GPU here): only the
    attributes the binding's output checks read."""

    def __init__(self, shape, dtype, contiguous=True, device="cuda:0", is_cuda=True):
        import torch
        self.shape, self.dtype, self._c = tuple(shape), dtype, contiguous
        self.device, self.is_cuda = torch.device(device), is_cuda

    def is_contiguous(self):
        return self._c


def test_output_checks():
    """Caller-supplied out= / lse= tensors must match exactly what the kernel
    writes through their raw pointers."""
    import torch
    dev = torch.device("cuda:0")
    ok = _FakeDeviceTensor((2, 3, 100, 64), torch.bfloat16)
    fa._check_out(ok, "out", (2, 3, 100, 64), torch.bfloat16, dev)
    with pytest.raises(ValueError):  # too small
        fa._check_out(_FakeDeviceTensor((2, 3, 99, 64), torch.bfloat16), "out", (2, 3, 100, 64), torch.bfloat16, dev)
    with pytest.raises(TypeError):  # wrong element size
        fa._check_out(_FakeDeviceTensor((2, 3, 100, 64), torch.float32), "out", (2, 3, 100, 64), torch.bfloat16, dev)
    with pytest.raises(ValueError):  # strided
        fa._check_out(_FakeDeviceTensor((2, 3, 100, 64), torch.bfloat16, contiguous=False), "out",
                      (2, 3, 100, 64), torch.bfloat16, dev)
    with pytest.raises(ValueError):  # host memory
        fa._check_out(_FakeDeviceTensor((2, 3, 100), torch.float32, device="cpu", is_cuda=False), "lse",
                      (2, 3, 100), torch.float32, dev)
    with pytest.raises(ValueError):  # another device
        fa._check_out(_FakeDeviceTensor((2, 3, 100), torch.float32, device="cuda:1"), "lse",
                      (2, 3, 100), torch.float32, dev)
    # real host tensors are refused outright
    x = torch.zeros(2, 3, 100, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa._check_out(x, "out", x.shape, x.dtype, dev)


def test_python_wrapper_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x[..., :32])


# ------------------------------------------------------------ key splits

def test_max_splits_matches_header():
    m = re.search(r"#define FA_MAX_SPLITS (\d+)", open(HEADER).read())
    assert fa.FA_MAX_SPLITS == int(m.group(1))


def test_static_scratch_size_matches_header():
    m = re.search(r"#define FA_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert fa.FA_STATIC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))


def test_split_static_checks_before_any_hip_call():
    """Argument errors and sizes beyond the static array are reported on the host
    (safe without a GPU: no HIP call is reached)."""
    f = fa.fa_fwd_split_static
    assert f(0, K, V, O, L, 1, 1, 64, 64, 0.125, 0, 1, 2, 0) == fa.FA_ERR_INVALID_ARG
    assert f(Q, K, V, O, L, 1, 1, 64, 64, float("nan"), 0, 1, 2, 0) == fa.FA_ERR_INVALID_ARG
    assert f(Q, K, V, O, L, 1, 1, 64, 64, 0.125, 0, 1, 0, 0) == fa.FA_ERR_INVALID_ARG
    assert f(Q, K, V, O, L, 1, 1, 64, 48, 0.125, 0, 1, 2, 0) == fa.FA_ERR_UNSUPPORTED
    assert f(Q, K, V, O, L, 1, 1, 64, 64, 0.125, 0, 1, fa.FA_MAX_SPLITS + 1, 0) == fa.FA_ERR_UNSUPPORTED
    # partials of B1 H2 N8192 D128 in 16 splits: 16*2*8192*129*4 bytes > 64 MiB
    big = dict(q=T, k=2 * T, v=3 * T, o=4 * T, lse=5 * T)
    need = fa.fa_fwd_split_workspace_bytes(1, 2, 8192, 128, 16)
    assert need > fa.FA_STATIC_SCRATCH_BYTES
    assert f(big["q"], big["k"], big["v"], big["o"], big["lse"], 1, 2, 8192, 128, 0.1, 0, 1, 16, 0) \
        == fa.FA_ERR_UNSUPPORTED


def test_split_workspace_bytes():
    ws = fa.fa_fwd_split_workspace_bytes
    assert ws(2, 8, 1024, 64, 4) == 4 * 2 * 8 * 1024 * 65 * 4
    assert ws(1, 1, 1, 128, 1) == 129 * 4
    for bad in ((0, 1, 1, 64, 1), (1, 0, 1, 64, 1), (1, 1, 0, 64, 1), (1, 1, 1, 0, 1), (1, 1, 1, 64, 0),
                (1, 1, 1, 64, -3)):
        assert ws(*bad) == 0
    assert ws(1 << 30, 1 << 30, 1 << 20, 128, 64) == 0  # overflows 64 bits


@pytest.mark.parametrize("shape,causal,n_cus,want", [
    ((2, 8, 1024, 64), 0, 256, 1),     # 64 workgroups, but 8 key tiles: too short to split
    ((2, 8, 1024, 64), 1, 256, 1),
    ((2, 8, 2048, 64), 0, 256, 2),     # 128 workgroups, 16 tiles -> 2 splits of 8 tiles
    ((4, 16, 4096, 128), 0, 256, 1),   # 1024 workgroups already fill the device
    ((1, 1, 128, 64), 0, 256, 1),      # one key tile: nothing to split
    ((1, 1, 4096, 128), 0, 256, 4),    # 16 workgroups want 16 splits; 32 tiles allow 4
    ((1, 1, 1 << 20, 128), 0, 256, 1),
    ((1, 1, 300000, 64), 0, 100000, 64),  # capped at FA_MAX_SPLITS
    ((1, 2, 8192, 128), 1, 256, 4),
])
def test_split_choose(shape, causal, n_cus, want):
    assert fa.fa_fwd_split_choose(*shape, causal, n_cus) == want


def test_split_choose_rejects_bad_arguments():
    assert fa.fa_fwd_split_choose(0, 1, 64, 64, 0, 256) == 0
    assert fa.fa_fwd_split_choose(1, 1, 64, 64, 2, 256) == 0
    assert fa.fa_fwd_split_choose(1, 1, 64, 64, 0, 0) == 0


WS = 0x60000000  # fake workspace address, clear of every tensor above
WS_BYTES = 1 << 28


def split_call(**kw):
    a = dict(GOOD, n_splits=3, ws=WS, ws_bytes=WS_BYTES)
    a.update(kw)
    return fa.fa_fwd_split(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["D"],
                           a["scale"], a["causal"], a["dtype"], a["n_splits"], a["ws"], a["ws_bytes"], 0)


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(B=0), dict(scale=float("nan")), dict(o=Q),           # the checks of fa_fwd
    dict(n_splits=0), dict(n_splits=-1), dict(ws=0), dict(ws=WS + 8),
    dict(ws_bytes=3 * 2 * 3 * 100 * 65 * 4 - 1), dict(ws=Q - 64), dict(ws=L - 256), dict(ws=O + 16),
])
def test_split_invalid_arguments(kw):
    # every one is rejected on the host before any HIP call, so this is safe without a GPU
    assert split_call(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(n_splits=65), dict(D=80), dict(D=96, dtype=0),
    # 2^22 workgroups pass fa_fwd's grid limit; two splits reach 2^23
    dict(B=1 << 12, H=1 << 8, N=1024, n_splits=2, q=T, k=2 * T, v=3 * T, o=4 * T, lse=5 * T, ws=6 * T,
         ws_bytes=1 << 62),
])
def test_split_unsupported(kw):
    assert split_call(**kw) == fa.FA_ERR_UNSUPPORTED


def test_large_grid_passes_fwd_checks():
    """The large-grid split case above is within fa_fwd's own limits."""
    assert check(B=1 << 12, H=1 << 8, N=1024, q=T, k=2 * T, v=3 * T, o=4 * T, lse=5 * T) == fa.FA_OK


PO, PL, MO, ML = 0x10000000, 0x20000000, 0x30000000, 0x40000000
MGOOD = dict(po=PO, pl=PL, P=3, rows=1000, D=64, o=MO, lse=ML, dtype=1)


def merge_call(**kw):
    a = dict(MGOOD)
    a.update(kw)
    return fa.fa_lse_merge(a["po"], a["pl"], a["P"], a["rows"], a["D"], a["o"], a["lse"], a["dtype"], 0)


@pytest.mark.parametrize("kw", [
    dict(po=0), dict(pl=0), dict(o=0), dict(lse=0), dict(P=0), dict(rows=0), dict(D=0), dict(dtype=3),
    dict(po=PO + 4), dict(o=MO + 8), dict(pl=PL + 2), dict(lse=ML + 1),
    dict(o=PO + 1024), dict(lse=PL + 64), dict(o=PL - 64), dict(lse=MO + 64),
])
def test_merge_invalid_arguments(kw):
    assert merge_call(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(P=1025), dict(D=4), dict(D=12), dict(D=520), dict(D=1024), dict(rows=1 << 40),
                                dict(P=1024, rows=1 << 24, D=512)])
def test_merge_unsupported(kw):
    assert merge_call(**kw) == fa.FA_ERR_UNSUPPORTED


# ------------------------------------------------------------ packed sequences

VQ, VK, VV, VO, VL, CQ, CK = (T * i for i in range(1, 8))
VGOOD = dict(q=VQ, k=VK, v=VV, o=VO, lse=VL, cq=CQ, ck=CK, n=3, H=4, tq=1000, tk=1200, maxq=500, D=128,
             scale=0.1, causal=1, dtype=1)


def vcheck(arch="gfx950", **kw):
    a = dict(VGOOD)
    a.update(kw)
    return fa.fa_check_varlen_args(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["n"], a["H"],
                                   a["tq"], a["tk"], a["maxq"], a["D"], a["scale"], a["causal"], a["dtype"], arch)


def test_varlen_good_arguments_pass():
    assert vcheck() == fa.FA_OK
    assert vcheck(arch=None) == fa.FA_OK
    for dt in (0, 1, 2):
        for D in (64, 128):
            for c in (0, 1):
                assert vcheck(dtype=dt, D=D, causal=c) == fa.FA_OK
    assert vcheck(maxq=1000) == fa.FA_OK and vcheck(n=1, maxq=1) == fa.FA_OK


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(lse=0), dict(cq=0), dict(ck=0),
    dict(n=0), dict(H=0), dict(tq=0), dict(tk=0), dict(D=0), dict(maxq=0), dict(maxq=1001),
    dict(scale=float("nan")), dict(causal=2), dict(dtype=5),
    dict(q=VQ + 8), dict(o=VO + 4), dict(lse=VL + 2), dict(cq=CQ + 2), dict(ck=CK + 1),
    dict(o=VQ + 256), dict(o=VK - 256), dict(lse=VV + 64), dict(lse=CQ), dict(o=CK - 16), dict(lse=VO + 1024),
])
def test_varlen_invalid_arguments(kw):
    assert vcheck(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(D=80), dict(D=512), dict(D=256, dtype=0), dict(tq=1 << 30, maxq=100), dict(tk=1 << 30), dict(H=1 << 20),
    dict(H=1 << 12, tq=1 << 24, maxq=100), dict(n=1 << 13, H=1 << 8, maxq=1000, tq=1 << 20),
])
def test_varlen_unsupported(kw):
    assert vcheck(**kw) == fa.FA_ERR_UNSUPPORTED


def test_varlen_unsupported_arch():
    assert vcheck(arch="gfx942") == fa.FA_ERR_UNSUPPORTED


def test_varlen_reports_invalid_args_before_any_hip_call():
    st = fa.fa_fwd_varlen(VQ, VK, VV, VO, VL, 0, CK, 3, 4, 1000, 1200, 500, 128, 0.1, 1, 1, 0)
    assert st == fa.FA_ERR_INVALID_ARG
    st = fa.fa_fwd_varlen(VQ, VK, VV, VO, VL, CQ, CK, 3, 4, 1000, 1200, 500, 80, 0.1, 1, 1, 0)
    assert st == fa.FA_ERR_UNSUPPORTED


# ------------------------------------------------------------ backward

BQ, BK, BV, BO, BDO, BL, BDQ, BDK, BDV, BWS = (T * i for i in range(1, 11))
BGOOD = dict(q=BQ, k=BK, v=BV, o=BO, do=BDO, lse=BL, dq=BDQ, dk=BDK, dv=BDV, B=2, H=3, N=500, D=128, scale=0.1,
             causal=1, dtype=1, ws=BWS, wsb=2 * 3 * 500 * 4)


def bcheck(arch="gfx950", **kw):
    a = dict(BGOOD)
    a.update(kw)
    return fa.fa_check_bwd_args(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                a["B"], a["H"], a["N"], a["D"], a["scale"], a["causal"], a["dtype"], a["ws"],
                                a["wsb"], arch)


def test_bwd_workspace_bytes():
    assert fa.fa_bwd_workspace_bytes(2, 3, 500, 128) == 2 * 3 * 500 * 4
    assert fa.fa_bwd_workspace_bytes(0, 3, 500, 128) == 0
    assert fa.fa_bwd_workspace_bytes(1 << 40, 1 << 30, 1, 64) == 0


def test_bwd_good_arguments_pass():
    assert bcheck() == fa.FA_OK and bcheck(arch=None) == fa.FA_OK
    for dt in (1, 2):
        for D in (32, 64, 96, 128, 160, 192, 224, 256):
            for c in (0, 1):
                assert bcheck(dtype=dt, D=D, causal=c) == fa.FA_OK
    for D in (64, 128):
        for c in (0, 1):
            assert bcheck(dtype=0, D=D, causal=c) == fa.FA_OK
    assert bcheck(scale=0.0) == fa.FA_OK and bcheck(scale=-2.0) == fa.FA_OK


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(do=0), dict(lse=0), dict(dq=0), dict(dv=0), dict(ws=0), dict(B=0), dict(N=0), dict(D=0),
    dict(scale=float("nan")), dict(causal=3), dict(dtype=4), dict(q=BQ + 2), dict(dk=BDK + 8), dict(ws=BWS + 4),
    dict(lse=BL + 1), dict(wsb=2 * 3 * 500 * 4 - 1), dict(dq=BO + 64), dict(dk=BQ - 64), dict(dv=BL - 16),
    dict(ws=BDO + 128), dict(dk=BDQ + 16), dict(ws=BDV - 1024),
])
def test_bwd_invalid_arguments(kw):
    assert bcheck(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(dtype=0, D=96), dict(dtype=0, D=256), dict(dtype=0, D=32), dict(dtype=0, D=160),
                                dict(D=48), dict(D=80), dict(D=288), dict(D=512),
                                dict(N=1 << 30),
                                dict(B=1 << 14, H=1 << 6, N=128 * 8, wsb=1 << 62)])
def test_bwd_unsupported(kw):
    assert bcheck(**kw) == fa.FA_ERR_UNSUPPORTED


def test_bwd_reports_invalid_args_before_any_hip_call():
    st = fa.fa_bwd(0, BK, BV, BO, BDO, BL, BDQ, BDK, BDV, 2, 3, 500, 128, 0.1, 1, 1, BWS, 12000, 0)
    assert st == fa.FA_ERR_INVALID_ARG
    st = fa.fa_bwd(BQ, BK, BV, BO, BDO, BL, BDQ, BDK, BDV, 2, 3, 500, 96, 0.1, 1, 0, BWS, 12000, 0)
    assert st == fa.FA_ERR_UNSUPPORTED


# ------------------------------------------------------------ FP8

F8 = dict(q=T, k=2 * T, v=3 * T, o=4 * T, lse=5 * T, B=2, H=3, N=1000, D=128, scale=0.1, qd=0.5, kd=2.0, vd=1.5,
          causal=0, ws=6 * T, wsb=2 * 3 * 128 * 1024)


def f8check(arch="gfx950", **kw):
    a = dict(F8)
    a.update(kw)
    return fa.fa_check_fp8_args(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["D"],
                                a["scale"], a["qd"], a["kd"], a["vd"], a["causal"], a["ws"], a["wsb"], arch)


def test_fp8_workspace_bytes():
    assert fa.fa_fwd_fp8_workspace_bytes(2, 3, 1000, 128) == 2 * 3 * 128 * 1024
    assert fa.fa_fwd_fp8_workspace_bytes(1, 1, 128, 64) == 64 * 128
    assert fa.fa_fwd_fp8_workspace_bytes(1, 0, 128, 64) == 0


def test_fp8_good_arguments_pass():
    assert f8check() == fa.FA_OK and f8check(arch=None) == fa.FA_OK
    for D in (32, 64, 96, 128, 160, 192, 224, 256):
        assert f8check(D=D, wsb=1 << 40) == fa.FA_OK
    assert f8check(D=64, causal=1, scale=-0.3, qd=-1.0) == fa.FA_OK


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(lse=0), dict(ws=0), dict(N=0), dict(scale=float("inf")), dict(qd=float("nan")),
    dict(vd=float("inf")), dict(scale=1e30, qd=1e30), dict(causal=2), dict(q=T + 4), dict(o=4 * T + 2),
    dict(lse=5 * T + 1), dict(ws=6 * T + 8), dict(wsb=2 * 3 * 128 * 1024 - 1), dict(o=T + 64),
    dict(ws=3 * T - 64), dict(lse=4 * T + 128),
])
def test_fp8_invalid_arguments(kw):
    assert f8check(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(D=80), dict(D=16), dict(D=288), dict(D=512), dict(N=1 << 24), dict(B=1 << 8, H=1 << 8)])
def test_fp8_unsupported(kw):
    assert f8check(**kw, wsb=1 << 62) == fa.FA_ERR_UNSUPPORTED
