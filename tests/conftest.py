import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size cases that take tens of seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding, on cuda:0; fails loudly when either is missing."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    from orthogonalizing_polynomial_cascade_amd import anvil
    anvil.load()
    return anvil
