import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """Skip-free guard: a gpu-marked test run without a GPU is an error, not a skip."""
    if not _gpu_available():
        pytest.fail("test marked gpu but torch sees no GPU")
    import torch
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def lib():
    """The loaded HIP library binding (fails loudly when it has not been built)."""
    from draft_sampling_verification_head_amd import binding
    return binding.load()
