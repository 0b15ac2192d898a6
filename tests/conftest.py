import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU-only check")


@pytest.fixture(scope="session")
def tiny_model():
    import oracle
    import synth
    d = synth.TINY
    W = synth.gen_weights(d, gain_std=0.1, weight_std=0.2, embed_std=1.0)
    return d, W, oracle.OracleModel(d, W)
