import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_sessionstart(session):
    # Load what is built; build only when nothing is (a fresh checkout).
    from fp8_blockwise_weight_amd import build

    build.ensure_built()


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; GPU tests fail loudly when it is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import fp8_blockwise_weight_amd as fq

    fq.load_library()
    return fq
