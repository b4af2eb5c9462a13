import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (seconds to a minute)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    yield oracle
    oracle.set_variant(0)


@pytest.fixture(scope="session", autouse=True)
def _built_library():
    """Build the HIP library in-tree if it is missing (normally built beforehand)."""
    import rejection_sampling_verify_10_amd as R
    if not os.path.exists(R.LIB_PATH):
        from rejection_sampling_verify_10_amd import build
        build.build()
