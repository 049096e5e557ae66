import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Build the CPU-side libraries if they are missing (the HIP library is built by build())."""
    from oracle import build as ob
    from datagen import build as db
    if not os.path.exists(ob.SO):
        ob.build()
    if not os.path.exists(db.HOST_SO):
        db.build_host()


_ensure_built()


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(12345)
