import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding on cuda:0.  Skips only when no GPU is visible; a GPU without the built
    library is an error, never a silent fallback."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_cache_pages_amd as pkv

    pkv.require_library()
    return pkv
