import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU oracle work")


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU and the built library are present; returns the binding module."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decoder_attention_amd as ga

    ga.load()  # raises if the library is missing: no silent fallback
    return ga
