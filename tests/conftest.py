import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def dev():
    """The GPU device for `gpu` tests; fails (not skips) when the library or GPU is missing, so a
    GPU run can never pass on a silent fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test requested but torch.cuda.is_available() is False")
    import quantized_state_space_amd as qs
    qs.load()  # raises if libqssm.so is missing
    return torch.device("cuda:0")
