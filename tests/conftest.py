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
def lib():
    """The HIP library binding.  On a machine with a GPU a missing or stale library is an
    error, never a skip: the product path has no fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from nvfp4_block_scaled_gather_amd import binding
    return binding.load()
