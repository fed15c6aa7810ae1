import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_threads():
    # the oracle uses the CPU share given to this process (OMP_NUM_THREADS when set)
    import oracle
    n = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    if n > 0:
        oracle.set_threads(n)
    yield
