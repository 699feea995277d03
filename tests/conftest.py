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
    lib = os.path.join(ROOT, "oracle", "liboracle_ln.so")
    srcs = [os.path.join(ROOT, "oracle", f) for f in ("ln_oracle.c", "ln_oracle.h")]
    stale = not os.path.exists(lib) or any(
        os.path.getmtime(s) > os.path.getmtime(lib) for s in srcs)
    oracle.build(force=stale)
    return oracle
