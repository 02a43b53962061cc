import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of host work)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The MFA binding, loaded from the in-tree build. Fails loudly if absent."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a GPU")
    import decode_attention_02_amd as mfa
    mfa.load()            # raises if libmfa.so is missing
    return mfa
