import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The built HIP library (fails loudly if it is missing or no GPU is present)."""
    if not gpu_available():
        pytest.fail("GPU test collected without a GPU: run with -m 'not gpu' on CPU hosts")
    import mixture_experts_ffn_softmax_amd as moe
    return moe
