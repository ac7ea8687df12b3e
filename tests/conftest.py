import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests of the HIP path")
    config.addinivalue_line("markers", "slow: large CPU work (oracle on big samples)")


@pytest.fixture(scope="session")
def libfa():
    """The in-tree libfa.so, built here with hipcc when it is missing (hipcc
    cross-compiles for gfx950 without a GPU).  A failed build fails every test
    that asks for the library; nothing is skipped."""
    import attention_fa_fwd_02_amd as fa
    if not os.path.exists(fa.lib_path()):
        from attention_fa_fwd_02_amd.build import build_library
        build_library()
    return fa.load_library()
