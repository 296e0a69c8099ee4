import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def _stamp(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Print (and flush) the name of every GPU case before it runs, so a run
    that dies on the device still names the case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        _stamp(f"[gpu-case] {request.node.nodeid}")
    yield
