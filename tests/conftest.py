import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")


@pytest.fixture(scope="session")
def oracle_mod():
    """The CPU oracle, built once per session if its library is missing or stale."""
    from oracle import build as obuild
    obuild.build(force=False)
    import oracle
    return oracle
