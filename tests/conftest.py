import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP binding, with the built library loaded; skips cleanly only when no GPU exists."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_causal_gqa_cpattn_amd as cp
    cp.load()  # raises if the library is missing: no fallback path exists
    return cp
