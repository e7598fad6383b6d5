import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests announce themselves before they run so a hang or a fault names its case.
    for item in items:
        if item.get_closest_marker("gpu") is not None:
            item.user_properties.append(("gpu", True))


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
