import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (seconds of oracle work)")


@pytest.fixture(scope="session")
def gpu():
    """The C-ABI library bound to device 0; fails loudly if the HIP build is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu-marked test run without a visible GPU")
    from dense_blas3_gemm_amd import Gemm
    g = Gemm(device=0)
    yield g
    g.close()
