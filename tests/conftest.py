import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (oracle at full size)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; skips without a GPU, fails loudly with a GPU but without the library."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import moe_grouped_gemm_e4m3_amd as fg

    fg.load_library()  # raises if the .so is missing or does not load
    return fg
