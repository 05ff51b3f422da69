import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libmoe")
    config.addinivalue_line("markers", "slow: full-size workloads (seconds to minutes)")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_ffn_04_amd import binding as libmoe
    libmoe.load()       # raises if the HIP library is missing
    return torch.device("cuda:0")
