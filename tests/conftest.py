import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding on cuda:0; fails loudly (never falls back) when the
    library is missing on a GPU machine."""
    if not _gpu_available():
        pytest.skip("no GPU")
    import compressed_kv_cache_absorbed_amd as mla
    mla.load()  # raises if the built library is absent
    return mla
