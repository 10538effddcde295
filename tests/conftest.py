import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build()
    return oracle


@pytest.fixture(scope="session")
def bkv():
    """The HIP library binding; on a GPU machine a missing library is an error, not a skip."""
    import kv_cache_eviction_continual_amd as pkg

    return pkg.lib()


@pytest.fixture(autouse=True)
def _debug_copies(request):
    """GPU tests compare the rotated observation rows that the scoring calls
    copy to the workspace when debug copies are on: turn the copies on for
    each GPU test and restore the previous setting after it."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    from kv_cache_eviction_continual_amd import bkv as b

    prev = b.bkv_set_debug_copies(True)
    yield
    b.bkv_set_debug_copies(prev)
