import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built libfd.so")
    config.addinivalue_line(
        "markers", "slow: large CPU-side work (full-size inputs)")


@pytest.fixture(scope="session")
def oracle_mod():
    """The fp64 oracle, built with gcc on first use if needed."""
    from oracle import oracle as o
    if not os.path.exists(o.LIB_PATH):
        from oracle import build as ob
        ob.build()
    return o
