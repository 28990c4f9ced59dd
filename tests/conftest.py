import gc
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a HIP device (MI355X) and the built libfcbo.so")
    config.addinivalue_line("markers", "slow: longer CPU test")


def _flush_case(item):
    # Name the case before any GPU step, so a run that ends abruptly still tells which one ran.
    print("\n[case] %s" % item.nodeid, flush=True)


@pytest.hookimpl(tryfirst=True)
def pytest_runtest_setup(item):
    if item.get_closest_marker("gpu") is not None:
        _flush_case(item)


def release_device_cache():
    """Hand the memory torch's caching allocator keeps from earlier tests back to
    the device.  The library allocates with hipMalloc directly, so the full-size
    tests, which need most of the device, call this first."""
    gc.collect()
    try:
        import torch

        if torch.cuda.is_available():
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    except ImportError:
        pass
