import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(autouse=True)
def _announce_gpu_test(request):
    # name every GPU case on the real stderr before it runs, so a run that ends abruptly
    # still says which case it was in
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"[test] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
