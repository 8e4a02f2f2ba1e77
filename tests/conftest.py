import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


try:  # the first import on a fresh machine is slow: take it at collection, not inside a test
    import torch  # noqa: F401
except Exception:  # pragma: no cover
    torch = None


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def pa_lib():
    """The HIP library through its Python binding; GPU tests only."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_prefix_cached_amd as pa
    pa.load()
    return pa
