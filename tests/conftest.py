import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; parity of the HIP path against the oracle")


@pytest.fixture(scope="session")
def coracle():
    """The C oracle loops, compiled once per session."""
    from oracle import cref
    cref.build()
    return cref
