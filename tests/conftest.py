import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")


@pytest.fixture(scope="session", autouse=True)
def _native_built():
    import __graft_entry__

    # the HIP libraries too: a library older than its sources is rebuilt,
    # so a test never runs code other than the tree's
    __graft_entry__.ensure_built("oracle", "synth", "synth_gpu", "qgemm", "qgemm_ceiling")
    yield
