import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (gfx950); runs through the C-ABI library")


def have_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """The loaded HIP library on cuda:0. Fails loudly if the library is missing."""
    if not have_gpu():
        pytest.skip("no GPU visible to torch")
    import block_sparse_decode_nvfp4_amd as m3s
    m3s.load()   # raises if libm3s.so is missing or not loadable
    return m3s
