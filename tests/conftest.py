import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _has_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is visible; the HIP library must then be built."""
    if not _has_gpu():
        pytest.skip("no GPU visible")
    import cholesky_spd_solve_amd as spd
    spd.load()  # raises if the HIP library is missing: no silent fallback
    return spd
