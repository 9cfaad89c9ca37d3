import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")


def pytest_collection_modifyitems(config, items):
    # keep a file's tests in their written order; GPU tests announce themselves
    pass


@pytest.fixture(autouse=True)
def _announce(request):
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield
