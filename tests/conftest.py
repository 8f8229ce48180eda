import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests run last inside each file's order is kept; nothing else to do.
    return


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; GPU tests fail loudly if it is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU (run with -m 'not gpu')")
    from lse_combine_amd import _lib

    return _lib.load()
