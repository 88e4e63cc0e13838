import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library, loaded on a GPU host.  Fails loudly if the
    extension is missing: there is no CPU fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import attention_backward_fa2_amd as fa
    fa.load_library()
    return fa
