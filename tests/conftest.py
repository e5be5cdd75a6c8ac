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
    """The oracle's C folds are built by __graft_entry__.build(); build them
    here too when missing so the CPU suite runs from a clean checkout."""
    so = os.path.join(ROOT, "oracle", "_fold.so")
    if not os.path.exists(so):
        from oracle import build as ob
        ob.build()
    yield
