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
    """Skips unless a ROCm GPU is visible; returns the loaded binding module."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_exact_attention_fa_amd as fa

    fa.load()  # raises if the HIP library was not built
    return fa
