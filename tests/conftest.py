import functools
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP kernels")


@functools.lru_cache(maxsize=1)
def gpu_visible() -> bool:
    try:
        import torch
        return bool(torch.cuda.is_available())
    except ImportError:
        return False


# Host-only tests that call an entry point with made-up device addresses and
# expect it to stop at the device check (TDG_ERR_NO_DEVICE): where a GPU is
# visible the call would launch on those addresses, so they are skipped there.
no_device_only = pytest.mark.skipif(gpu_visible(), reason="fake device pointers would reach a real GPU")
