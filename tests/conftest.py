import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def gemm_tol(k: int, ref_absmax: float) -> float:
    """Acceptance bound for bf16-in / fp32-accumulate GEMM outputs:
    max |gpu - ref| <= 2e-2 * sqrt(K / 4096) * max |ref|."""
    return 2e-2 * (k / 4096.0) ** 0.5 * ref_absmax


@pytest.fixture(scope="session")
def tol():
    return gemm_tol
