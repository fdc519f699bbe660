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
    """The device-side test context: skips when no GPU is visible, fails loudly
    when a GPU is visible but the HIP library is not built or not loadable."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import selective_scan_recurrence_amd as ssm
    ssm.load()  # raises if libssm.so is missing
    return ssm
