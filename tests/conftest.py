import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="session", autouse=True)
def _library_built():
    """Build libtpmlp.so once if it is missing (an existing build is used as is)."""
    from tensor_transformer_layer_fwd_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from tensor_transformer_layer_fwd_amd import build
        build.build()
