import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of oracle or GPU time)")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound on cuda:0; fails loudly (never skips) without a GPU."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    import kv_block_selection_amd as kbs
    kbs.load()  # raises if libsparda.so is missing
    return kbs
