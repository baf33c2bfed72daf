import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0; skips when this machine has no GPU at all.

    On a machine with a GPU a missing or unloadable library is an error, not a skip.
    """
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    from allgather_gemm_persistent_amd import binding
    return binding.load()
