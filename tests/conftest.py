import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large-shape parity case (still GPU-only)")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0.  Fails (does not skip) when a GPU is
    present but the library cannot be loaded."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import precision_attention_forward_amd as paf
    paf.load_library()          # raises if the shared library is missing
    return paf


def pytest_sessionfinish(session, exitstatus):
    # stop the oracle's worker processes, if a parity check started them
    mod = sys.modules.get("oracle_pool")
    if mod is not None:
        mod.shutdown()
