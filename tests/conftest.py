import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes on the CPU side)")


@pytest.fixture(scope="session")
def built_library():
    """libfluxmi.so, compiled first (hipcc, gfx950; no GPU needed) when a fresh
    checkout has none yet."""
    import tile_gemm_communication_amd as fm
    from tile_gemm_communication_amd import build
    if not os.path.exists(fm.LIB_PATH) or not os.path.exists(build.RESOURCES):
        build.build(verbose=False)
    return fm.lib()


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle
    return _oracle.load()
