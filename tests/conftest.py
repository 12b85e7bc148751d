import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an AMD Instinct GPU and the built libmapflow.so")


@pytest.fixture(scope="session")
def gpu():
    """The GPU device; a gpu-marked test fails (never skips) without one."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import cross_model_sparse_amd as mf
    mf.load()  # raises if libmapflow.so is missing: no fallback path exists
    return torch.device("cuda:0")
