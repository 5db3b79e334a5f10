import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_sessionstart(session):
    # The C oracle is single-threaded; independent tokens and experts are
    # spread over the host's cores (results do not depend on the count).
    import oracle
    oracle.set_threads(min(os.cpu_count() or 1, 16))
