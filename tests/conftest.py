import os
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) and the built libgla.so")


@pytest.fixture(scope="session")
def gla():
    """The HIP binding; fails loudly when the library or the GPU is missing."""
    import torch
    import gated_linear_attention_gla_amd as pkg

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    pkg.load_library()
    from gated_linear_attention_gla_amd import _binding
    return _binding
