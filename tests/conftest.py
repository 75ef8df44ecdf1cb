import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libmla")
    config.addinivalue_line("markers", "slow: long CPU-side case")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def mla():
    """The product binding; on a GPU machine its absence is an error, not a skip."""
    import mla_latent_kv_16_amd as m
    m.load()  # raises if libmla.so is missing
    return m


@pytest.fixture(scope="session")
def gpu_lib():
    """The same check as `mla`, for tests that import the package under that name."""
    import mla_latent_kv_16_amd as pkg
    return pkg.load()
