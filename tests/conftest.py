import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding on cuda:0.  Fails (never skips, never falls back) if
    the GPU or the built library is missing."""
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU (torch.cuda.is_available() is False)")
    from memory_bound_gemv_row_amd import binding

    binding.load()
    return binding
