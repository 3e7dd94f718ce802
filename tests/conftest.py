import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_built():
    """Build the gcc helpers (and the HIP library) only when nothing is built yet."""
    import oracle
    import synth

    if not os.path.exists(synth._LIB_PATH):
        synth.build()
    if not os.path.exists(oracle._LIB_PATH):
        oracle.build()


_ensure_built()


@pytest.fixture(scope="session")
def gpu_available():
    import torch

    return torch.cuda.is_available()
