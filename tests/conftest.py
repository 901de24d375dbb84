import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests"), os.path.join(ROOT, "tests", "golden")):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity of the HIP path")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle


@pytest.fixture(scope="session")
def qll_gpu():
    """The HIP library's Python binding on cuda:0.  A GPU test never falls
    back to anything: if the device is there, the library must load."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import quantized_linear_layer_amd as qll
    qll.load()  # raises if libqll.so is missing or broken
    return qll
