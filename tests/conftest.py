import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test (exhaustive sweeps)")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def fgq_gpu():
    """The GPU binding; a GPU test fails loudly (not skips) if the library is missing."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import fine_grained_fp8_quant_amd as fgq
    fgq.load_library()  # raises if the HIP library is not built
    return fgq
