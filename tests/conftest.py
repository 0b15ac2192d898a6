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


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    if not _gpu_available():
        pytest.skip("no GPU")
    import streaming_tts_decode_amd as qt
    qt.lib()  # raises if the HIP library is missing
    return qt


@pytest.fixture(scope="session")
def full_weights():
    import synth
    return synth.gen_weights(synth.FULL)


@pytest.fixture(scope="session")
def orc_full(full_weights):
    import oracle
    import synth
    return oracle.OracleModel(synth.FULL, full_weights)


@pytest.fixture(scope="session")
def orc_full_i8(full_weights):
    import oracle
    import synth
    return oracle.OracleModel(synth.FULL, full_weights, int8=True)


@pytest.fixture(scope="session")
def full_pm(gpu, full_weights):
    import synth
    from streaming_tts_decode_amd.runtime import PackedModel
    pm = PackedModel(synth.FULL, full_weights, int8=False)
    yield pm
    pm.close()


@pytest.fixture(scope="session")
def full_pm_i8(gpu, full_weights):
    import synth
    from streaming_tts_decode_amd.runtime import PackedModel
    pm = PackedModel(synth.FULL, full_weights, int8=True)
    yield pm
    pm.close()


@pytest.fixture(scope="session")
def small_weights():
    import synth
    return synth.gen_weights(synth.SMALL, gain_std=0.1)


@pytest.fixture(scope="session")
def orc_small(small_weights):
    import oracle
    import synth
    return oracle.OracleModel(synth.SMALL, small_weights)


@pytest.fixture(scope="session")
def small_pm(gpu, small_weights):
    import synth
    from streaming_tts_decode_amd.runtime import PackedModel
    pm = PackedModel(synth.SMALL, small_weights, int8=False)
    yield pm
    pm.close()
