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


# ---------------------------------------------------------------- GPU fixtures

class _DeviceWeights:
    """Device copies of the synthetic layers, generated on the GPU once per session."""

    def __init__(self):
        self.layers = {}
        self.lm = None

    def layer(self, wl, l):
        from datagen import device as D
        key = (wl.family, wl.I, wl.shard, wl.n_shards, l)
        if key not in self.layers:
            self.layers[key] = D.make_layer(wl, l)
        return self.layers[key]

    def layer_fp8(self, wl, l):
        from datagen import device as D
        key = ("fp8", wl.family, wl.I, l)
        if key not in self.layers:
            self.layers[key] = D.make_layer_fp8(wl, l)
        return self.layers[key]

    def lmhead(self, wl):
        from datagen import device as D
        if self.lm is None:
            self.lm = D.make_lmhead(wl)
        return self.lm


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def dw(gpu):
    return _DeviceWeights()
