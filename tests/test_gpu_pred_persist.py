"""The one-launch code predictor (QT_PREDICTOR=persistent at model load; every
predictor step of a frame in one launch of 256 blocks) against the oracle at the
full model's shapes: the predictor-only workload, B=32 graph frames, and INT8
weights.  The default frame runs the predictor as a chain of launches; both compute
the same definition and are held to the same parity gates."""
import dataclasses
import os

import numpy as np
import pytest

import synth
from tests.gpu_cases import run_frames

pytestmark = pytest.mark.gpu


def _load(weights, int8):
    from streaming_tts_decode_amd.runtime import PackedModel
    os.environ["QT_PREDICTOR"] = "persistent"
    try:
        return PackedModel(synth.FULL, weights, int8=int8)
    finally:
        del os.environ["QT_PREDICTOR"]


@pytest.fixture(scope="module")
def pm_persist(gpu, full_weights):
    pm = _load(full_weights, False)
    yield pm
    pm.close()


def test_persistent_predictor_runs_as_one_launch(pm_persist):
    from streaming_tts_decode_amd.runtime import setup_workload
    w = dataclasses.replace(synth.WORKLOADS["C3"], frames=1)
    dec, _ = setup_workload(w, pm_persist)
    dec.set_inputs(talker_in=synth.frame_inputs(w)["talker_in"][0])
    rec = dec.trace("full")
    kinds = [k for _, k, _, _ in rec]
    assert kinds.count("predictor") == 1
    assert kinds.count("attn_pred") == 0 and kinds.count("embed") == 0
    assert int(dec.status.item()) == 0
    dec.close()


def test_persistent_predictor_c1(pm_persist, orc_full):
    run_frames(pm_persist, orc_full, synth.WORKLOADS["C1"], check=[0])


def test_persistent_predictor_b32_graph(pm_persist, orc_full):
    w = dataclasses.replace(synth.WORKLOADS["C4"], frames=3)
    L = w.lengths()
    run_frames(pm_persist, orc_full, w, check=[int(np.argmin(L)), int(np.argmax(L))],
               use_graph=True)


def test_persistent_predictor_int8(gpu, full_weights, orc_full_i8):
    pm = _load(full_weights, True)
    try:
        w = dataclasses.replace(synth.WORKLOADS["C5B1"], frames=2)
        run_frames(pm, orc_full_i8, w, check=[0], use_graph=True)
    finally:
        pm.close()
