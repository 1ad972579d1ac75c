import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built libkvc")


def _gpu_present() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """The HIP device and the loaded library. Fails (not skips) when a GPU is
    present but the native library is missing, so GPU runs never pass on a
    fallback."""
    if not _gpu_present():
        pytest.skip("no GPU visible")
    import kv_cache_append_amd as kvc
    kvc.load()  # raises if libkvc.so is not built
    import torch
    return torch.device("cuda:0")
