import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: long CPU test (still part of the CPU suite)")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built on first use)."""
    import oracle
    return oracle.default()


@pytest.fixture(scope="session")
def hip():
    """The HIP library's Python binding, on a GPU; skips without one."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_gemm_amd as bs
    bs.lib()  # raises if the HIP library is missing
    return bs
