import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload checks")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The HIP library through its Python binding; fails loudly when it is missing on a GPU machine."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import transformer_attention_sdpa_amd as sdpa_amd
    sdpa_amd.load()          # raises if the shared library was not built
    return sdpa_amd
