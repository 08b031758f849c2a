import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def orc():
    """The oracle library; ORACLE_LIB may name a planted-mistake copy (used only
    by the mutation test, which expects the pins to fail on such a copy)."""
    import oracle

    path = os.environ.get("ORACLE_LIB")
    return oracle.Oracle(path) if path else oracle.get()
