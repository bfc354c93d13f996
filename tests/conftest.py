import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU oracle check")


def oracle_threads():
    """Threads the oracle's attention may use: the host's CPU share (the
    OMP_NUM_THREADS setting where there is one), at most 16."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


@pytest.fixture(scope="session", autouse=True)
def _oracle_threads():
    from oracle import flux3_oracle as O
    O.THREADS = oracle_threads()
    yield


@pytest.fixture(scope="session")
def repo_root():
    return ROOT
