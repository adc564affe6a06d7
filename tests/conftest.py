import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def relerr(x, ref):
    """Max-abs error normalised by the reference's max-abs value (the
    tolerance norm used throughout: max_i |x_i - ref_i| / max_i |ref_i|)."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle
