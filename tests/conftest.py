import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
    except ImportError:
        return False
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def dev():
    """The GPU device; skips only when the machine has no GPU at all. With a
    GPU present, a missing or unloadable HIP library is a failure."""
    if not gpu_available():
        pytest.skip("no GPU on this machine")
    import torch
    import binary_rank_linear_amd as blr
    blr.load()  # raises if the library is missing
    return torch.device("cuda:0")
