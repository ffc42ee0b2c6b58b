import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _torch_device_first(request):
    """GPU tests start torch's device runtime before the library's first HIP call, so the
    device memory and streams the tests hand to the library come from one initialised
    runtime."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch
        torch.cuda.init()
    yield
