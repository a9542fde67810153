import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, on a machine with a GPU.  Fails loudly when the GPU is
    there but the library is not built or does not load."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    import dit_adaln_row_amd as dn
    dn.load()  # raises if the HIP library is missing
    return dn
