import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X) and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU-side case")


@pytest.fixture(scope="session")
def ora():
    import oracle
    oracle.build()
    return oracle
