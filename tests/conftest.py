import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """Fails (does not skip) when no GPU is visible: GPU tests are only ever
    selected where a GPU is meant to be present."""
    import torch

    assert torch.cuda.is_available(), "GPU test selected but no GPU is visible"
    return torch.device("cuda:0")
