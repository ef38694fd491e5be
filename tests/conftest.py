import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large inputs (seconds to minutes)")


def _ensure_built():
    """Build the host-side C libraries only if nothing is built yet."""
    import graphgen
    import oracle
    if not os.path.exists(graphgen._LIB):
        graphgen.build()
    if not os.path.exists(oracle._LIB):
        oracle.build()


_ensure_built()


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
