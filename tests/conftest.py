import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded on a GPU.  GPU tests fail (not skip) if it is missing."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    from long_reasoning_decode_amd import triattn
    triattn.load()
    return triattn
