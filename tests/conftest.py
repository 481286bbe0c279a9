import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU-side inputs")


@pytest.fixture(scope="session", autouse=True)
def _host_helpers_built():
    """The oracle and the graph generator are small C libraries built with gcc."""
    import graphgen
    import oracle
    if not os.path.exists(oracle._LIB):
        oracle.build(force=True)
    if not os.path.exists(graphgen._LIB):
        graphgen.build(force=True)
    yield
