"""Full-size parity of the HIP decode frame against the CPU oracle on the five
workloads (seeded synthetic weights and inputs at the real model shapes):

  C1  predictor-only frame, B=1                       (all outputs checked)
  C2  Talker step, B=1, 256 prefilled positions      (all outputs checked)
  C3  full frame, B=6, ragged KV 64..512, 12 frames  (all 6 sessions x 12 frames)
  C4  full frame, B=32, ragged KV 512..2048, 25 frames, one graph replayed
                                  (shortest, median and longest session x 25 frames)
  C5  INT8 weight-only, B=1 and B=32, graph, 25 frames
                                  (B=32: shortest, median and longest session)

The GPU always runs the whole batch in the benchmarked launch configuration;
the slow oracle recomputes the sessions listed.  The shortest session of a
ragged batch has the fewest attention splits and merge rounds, the longest the
most, so both ends of the split logic are compared with the oracle at every
frame."""
import numpy as np
import pytest

import synth
from tests.gpu_cases import run_frames

pytestmark = pytest.mark.gpu


def spread(lengths):
    """Sessions with the shortest, the median and the longest cached length."""
    order = np.argsort(lengths, kind="stable")
    return [int(order[0]), int(order[len(order) // 2]), int(order[-1])]


def test_c1_predictor_frame(full_pm, orc_full):
    run_frames(full_pm, orc_full, synth.WORKLOADS["C1"], check=[0])


def test_c2_talker_step(full_pm, orc_full):
    run_frames(full_pm, orc_full, synth.WORKLOADS["C2"], check=[0])


def test_c3_full_frame_b6(full_pm, orc_full):
    w = synth.WORKLOADS["C3"]
    run_frames(full_pm, orc_full, w, check=list(range(w.batch)))


def test_c4_full_frame_b32_graph(full_pm, orc_full):
    w = synth.WORKLOADS["C4"]
    run_frames(full_pm, orc_full, w, check=spread(w.lengths()), use_graph=True)


def test_c5_int8_b1_graph(full_pm_i8, orc_full_i8):
    w = synth.WORKLOADS["C5B1"]
    run_frames(full_pm_i8, orc_full_i8, w, check=[0], use_graph=True)


def test_c5_int8_b32_graph(full_pm_i8, orc_full_i8):
    w = synth.WORKLOADS["C5B32"]
    run_frames(full_pm_i8, orc_full_i8, w, check=spread(w.lengths()), use_graph=True)
