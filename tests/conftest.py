import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_setup(item):
    # name the case before any GPU work starts, so that a fault can be attributed
    if item.get_closest_marker("gpu") is not None:
        print(f"\n[gpu case] {item.nodeid}", flush=True)


@pytest.fixture(autouse=True)
def _float32_default():
    """Every test starts from torch's float32 default; a test that needs float64 says so in its
    tensors, and nothing it changes leaks into later tests."""
    try:
        import torch
    except ImportError:
        yield
        return
    torch.set_default_dtype(torch.float32)
    yield
    torch.set_default_dtype(torch.float32)


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build()
    return oracle
