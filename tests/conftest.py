import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _have_gpu() -> bool:
    try:
        import torch
        return bool(torch.cuda.is_available())
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """Skip-free guard: a GPU test run without a GPU is an error, not a skip."""
    if not _have_gpu():
        pytest.fail("this test needs a GPU (run with -m 'not gpu' on a CPU-only host)")
    import torch
    return torch.device("cuda:0")
