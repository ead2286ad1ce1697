import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="session")
def dev():
    """cuda:0 with the in-tree liblwg.so loaded; GPU tests fail (not skip) without them."""
    import torch
    import layernorm_window_gather_amd as lwg
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    lwg.library()
    return torch.device("cuda", 0)
