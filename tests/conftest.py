import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")

import pytest


@pytest.fixture(scope="session")
def native():
    """The ctypes binding, with libpagedkv.so built in-tree if it is not there yet."""
    from paged_kv_cache_320_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from paged_kv_cache_320_amd import build
        build.build()
    _lib.lib()
    return _lib


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False
