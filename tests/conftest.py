import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU-only oracle check")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library and a CUDA device; skips when no GPU is visible."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import sparse_kv_cache_ts_amd as ts
    ts.load()          # raises if the built library is missing
    return ts
