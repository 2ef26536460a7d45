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
    """The loaded C-ABI library on a machine with a GPU; fails loudly when it is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("a gpu-marked test ran without a visible GPU")
    from quantized_routed_expert_moe_amd import lib

    return lib.load()
