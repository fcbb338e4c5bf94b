import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle run")


@pytest.fixture(scope="session")
def gpu():
    """The GPU library handle; fails (does not skip) when no GPU is visible."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a visible GPU")
    from entropy_gated_kv_amd import lib
    return lib.load()
