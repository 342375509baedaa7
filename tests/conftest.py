import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libkvt.so")


@pytest.fixture(scope="session")
def gpu():
    """The device for GPU tests.  A gpu-marked test never falls back to the CPU: without a GPU
    it fails, loudly."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("this test needs a GPU (run it with -m gpu on an MI355X)")
    return torch.device("cuda:0")
