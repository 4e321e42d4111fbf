import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library, loaded through its C-ABI binding; the GPU tests fail (not skip)
    when a GPU is present but the library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_megakernel_amd as mk
    return mk
