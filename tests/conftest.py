import os
import sys

import numpy as np
import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def rel_err(got, ref, valid_mask=None) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rms(r)), rms over the compared (valid) entries."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if valid_mask is not None:
        g = g[valid_mask]
        r = r[valid_mask]
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(g - r) / den))


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build()
    return oracle
