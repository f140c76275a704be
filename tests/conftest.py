import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built C-ABI library, for tests marked gpu; fails loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test run without a visible GPU")
    import kv_cache_vector_fa_amd as fa
    fa.load()
    return fa
