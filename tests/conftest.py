import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0.  Skips only when no GPU is present;
    on a GPU machine a missing or broken library is an error, never a skip."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU present")
    import bit_quantized_moe_q2_amd as ds4q
    ds4q.load()          # raises if libds4q.so is missing
    return ds4q
