import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running oracle check")


@pytest.fixture(scope="session")
def libssa():
    """The built C-ABI library (built in-tree first if it is missing).  SSA_HOST_CHECK_LIB
    names another build of the same ABI to test instead: the host-sanitizer build of the
    argument checks (tests/test_host_sanitizers.py)."""
    from block_sparse_top_ssa_amd import _lib
    other = os.environ.get("SSA_HOST_CHECK_LIB")
    if other:
        return _lib.load(other)
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_top_ssa_amd import build
        build.build()
    return _lib.load()


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False
