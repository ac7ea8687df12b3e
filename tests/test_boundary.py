"""CPU tests of the C-ABI boundary: the library loads, exports every symbol the
header declares, and every argument error is reported on the host before any
HIP call (no compute calls here)."""
import os
import re

import pytest

import attention_fa_fwd_02_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.lib_path()), reason="libfa.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = fa.load_library()
    names = declared_functions()
    assert set(names) == {"fa_fwd", "fa_check_args", "fa_status_string", "fa_abi_version"}
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
    dict(D=32), dict(D=96), dict(D=256), dict(N=1 << 30), dict(B=1 << 20, H=1 << 10, N=1 << 7),
    dict(B=1 << 15, H=1 << 8, N=257),
])
def test_unsupported(kw):
    assert check(**kw) == fa.FA_ERR_UNSUPPORTED


def test_unsupported_arch():
    assert check(arch="gfx942:sramecc+:xnack-") == fa.FA_ERR_UNSUPPORTED
    assert check(arch="gfx1100") == fa.FA_ERR_UNSUPPORTED


def test_fwd_reports_invalid_args_before_any_hip_call():
    # NULL q: rejected on the host, so this is safe without a GPU
    st = fa.fa_fwd(0, K, V, O, L, 1, 1, 64, 64, 0.125, 0, 1, 0)
    assert st == fa.FA_ERR_INVALID_ARG
    st = fa.fa_fwd(Q, K, V, O, L, 1, 1, 64, 48, 0.125, 0, 1, 0)
    assert st == fa.FA_ERR_UNSUPPORTED


def test_python_wrapper_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x[..., :32])
