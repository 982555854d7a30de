import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size oracle comparison (tens of seconds)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library; a GPU test without it fails loudly."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    from speculative_decode_verification_router_amd import binding

    return binding.load()
