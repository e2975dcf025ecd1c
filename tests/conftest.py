import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path through the C-ABI")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def gpu():
    """Skip when there is no GPU; on a GPU machine, the library must load
    (a missing build is an error, not a skip)."""
    if not gpu_available():
        pytest.skip("no GPU on this machine")
    from block_sparse_masked_spec_amd import binding
    binding.load()  # raises if libsparse_attn.so is missing
    return binding
