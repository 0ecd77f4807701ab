"""Shared test setup: the `gpu` marker and lazy builds of what tests load."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its binding; fails loudly if it is not built."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_rope_amd as ar
    ar.load()  # raises if the shared library is missing
    return ar
