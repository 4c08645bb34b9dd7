import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C-ABI")
    config.addinivalue_line("markers", "slow: long-running (large shapes)")


def _cuda_ok():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def dev():
    """The GPU (HIP) device for parity tests; skips where there is none."""
    if not _cuda_ok():
        pytest.skip("no GPU")
    import torch
    import fine_grained_block_amd as fgb
    fgb.lib()  # fail loudly if the library is missing
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Print (and flush) which GPU case is about to run, so a failure names it."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    yield
