import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X GPU (gfx950)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=not os.path.exists(
        os.path.join(ROOT, "oracle", "liboracle_ln.so")))
    return oracle
