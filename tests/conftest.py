import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size case, minutes of CPU work")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, after checking that a GPU is present. GPU tests fail
    (they are not skipped) when the library or the device is missing."""
    import torch

    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import dynamic_quantized_gemm_amd as dq

    dq.load()  # raises if libdqip.so is missing
    return dq
