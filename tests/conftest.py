import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# outputs the binding allocates start as NaN (integers as INT32_MAX) in the
# tests, so that an element the library leaves unwritten fails a comparison
os.environ.setdefault("GNN_POISON_OUTPUTS", "1")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host time)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture
def live(pytestconfig):
    """print() that bypasses pytest's output capture, for progress lines of
    long tests (each line is flushed as it is written)."""
    cm = pytestconfig.pluginmanager.getplugin("capturemanager")

    def out(*a):
        if cm is None:
            print(*a, flush=True)
            return
        with cm.global_and_fixture_disabled():
            print(*a, flush=True)
    return out
