import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle work")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP binding with a GPU present; fails loudly when the library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from cem_jepa_predictor_amd import _lib

    return _lib.load()
