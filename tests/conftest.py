import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU tests")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; skips nothing: a GPU test without
    a GPU or without the built library fails loudly."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    from nf4_weight_streamed_amd import lib

    return lib
