import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library through its C ABI")


@pytest.fixture(scope="session")
def oracle():
    import oracle as o
    o.lib()
    return o


def gpu_available() -> bool:
    import torch
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def fp4():
    """The product library, loaded for GPU tests.  A GPU test without a GPU or
    without the built library fails loudly: there is no fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import nvfp4_bit_microscaled_amd as m
    m.load()
    return m
