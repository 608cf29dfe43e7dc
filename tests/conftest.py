import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


@pytest.fixture(autouse=True)
def _dispatcher_restored():
    """Whatever a test forced through rmsnorm_tune (a kernel variant, a grid
    cap) is undone when it ends, even when it fails."""
    yield
    from row_wise_normalization_rmsnorm_amd import binding
    if binding._lib is not None:
        binding.tune(None, 0)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long test (CPU or GPU), skipped unless RMSNORM_SLOW_TESTS=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("RMSNORM_SLOW_TESTS") == "1":
        return
    skip = pytest.mark.skip(reason="slow test; set RMSNORM_SLOW_TESTS=1")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)
