import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: larger CPU cases")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.default()


@pytest.fixture(scope="module")
def oracle_threads():
    """The oracle spread over the host's cores (at most 16) for the module:
    its outputs are independent, so the thread count does not change a bit."""
    import oracle
    lib = oracle.default()
    lib.set_threads(max(1, min(16, len(os.sched_getaffinity(0)))))
    yield lib
    lib.set_threads(1)
