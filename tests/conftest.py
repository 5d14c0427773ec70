import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


@pytest.fixture(scope="session", autouse=True)
def _host_libs():
    """Build the host-only helper libraries (gcc, seconds) if they are absent."""
    import corpus
    import oracle
    corpus.build(force=False)
    oracle.build(force=False)
