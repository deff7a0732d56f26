import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")


def _gpu_present() -> bool:
    try:
        import torch
    except Exception:
        return False
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def gpu():
    """Skips only when no GPU is visible; a missing HIP library still fails loudly."""
    if not _gpu_present():
        pytest.skip("no GPU visible")
    import torch
    return torch.device("cuda:0")
