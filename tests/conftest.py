import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU")


@pytest.fixture(scope="session")
def oracle():
    """The built CPU oracle (compiled from oracle/sgemm_oracle.c when missing or stale)."""
    from oracle import default_oracle

    return default_oracle()
