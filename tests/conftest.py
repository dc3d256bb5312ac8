import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """Build the CPU oracle once if it is not built yet."""
    from oracle import build as oracle_build
    if not os.path.exists(oracle_build.LIB):
        oracle_build.build()
    yield


@pytest.fixture(scope="session")
def hip_lib():
    """The HIP library, built here only if nothing is built yet."""
    from scaled_dot_product_12_amd import build as lib_build
    if not os.path.exists(lib_build.LIB):
        lib_build.build()
    import scaled_dot_product_12_amd as attn
    return attn
