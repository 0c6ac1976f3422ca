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


@pytest.fixture(scope="session")
def full_weights(lib):
    """The 288-expert, H=4096, I=2048 NVFP4 expert set (4.08 GB) of the full-size
    workloads, packed once per session and shared by every full-size GPU test."""
    from nvfp4_block_scaled_gather_amd import layer as L
    from nvfp4_block_scaled_gather_amd import workloads as W
    print("packing the full expert set", flush=True)
    wl = W.make_workload("decode1")
    w13 = L.pack_expert_weights(wl.w13, wl.E, 2 * wl.I, wl.H)
    print("w13 packed", flush=True)
    w2 = L.pack_expert_weights(wl.w2, wl.E, wl.H, wl.I)
    print("w2 packed", flush=True)
    return w13, w2
