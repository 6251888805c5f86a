import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def lib():
    """The C library, built first only if no build is present."""
    from sliding_window_gqa_varlen_amd import binding
    if not os.path.exists(binding.library_path()):
        from sliding_window_gqa_varlen_amd import build
        build.build()
    return binding.load_library()


@pytest.fixture(scope="session")
def gpu(lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")
