"""Host-only checks of the lockstep scheduler's C ABI (include/qt_sched.h): the
grouping rule, the buffer sizes and argument errors.  No GPU is needed: these
calls return before touching the device.

Grouping rule under test (decomputer.nl article on Qwen3-TTS serving, section 5:
graphs for a fixed set of batch sizes, oversize ready groups split over several
turns; "Qwen3-TTS Native v0.3.0", What changed: first frames bypass the lockstep
rendezvous): classes never mix, lower classes first, each class cut into groups
of the largest captured size plus one remainder, each group on the smallest size
that holds it."""
import math

import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def qt():
    import streaming_tts_decode_amd as qt
    qt.lib()
    return qt


def check_plan(cls, buckets, group_of, group_bucket):
    """Properties every grouping must have, plus the exact group sizes."""
    n = len(cls)
    bmax = buckets[-1]
    assert len(group_of) == n
    groups = {}
    for i, g in enumerate(group_of):
        groups.setdefault(g, []).append(i)
    assert sorted(groups) == list(range(len(group_bucket)))
    last_cls = -1
    for g in range(len(group_bucket)):
        members = groups[g]
        cs = {cls[i] for i in members}
        assert len(cs) == 1, f"group {g} mixes classes {cs}"
        c = cs.pop()
        assert c >= last_cls, "classes must run in ascending order"
        last_cls = c
        size = len(members)
        assert 1 <= size <= bmax
        assert group_bucket[g] == min(b for b in buckets if b >= size)
    for c in set(cls):
        idx = [i for i in range(n) if cls[i] == c]
        gs = [group_of[i] for i in idx]
        assert gs == sorted(gs), "within a class, sessions fill groups in input order"
        sizes = [gs.count(g) for g in sorted(set(gs))]
        m = len(idx)
        assert len(sizes) == math.ceil(m / bmax)
        assert sizes == [bmax] * (m // bmax) + ([m % bmax] if m % bmax else [])


@pytest.mark.parametrize("buckets", [[1], [4], [1, 2, 4, 8, 16, 32], [8, 32], [3, 5, 6]])
@pytest.mark.parametrize("n", [0, 1, 5, 8, 31, 32, 33, 70])
def test_plan_properties(qt, buckets, n):
    rng = np.random.default_rng(1000 + n)
    for trial in range(3):
        cls = rng.integers(0, 4, size=n).tolist() if trial else [2] * n
        group_of, group_bucket = qt.qt_sched_plan(cls, buckets)
        check_plan(cls, buckets, group_of, group_bucket)


def test_plan_worked_cases(qt):
    # 11 running sessions on {1,2,4,8}: one full group of 8 and a remainder of 3 on size 4
    g, b = qt.qt_sched_plan([2] * 11, [1, 2, 4, 8])
    assert g == [0] * 8 + [1] * 3 and b == [8, 4]
    # two first-frame sessions among running ones are decoded first, in their own group
    g, b = qt.qt_sched_plan([2, 0, 2, 2, 0], [1, 2, 4])
    assert g == [1, 0, 1, 1, 0] and b == [2, 4]
    # forced and free-running sessions never share a call
    g, b = qt.qt_sched_plan([3, 2, 3], [4])
    assert g == [1, 0, 1] and b == [4, 4]
    # 33 sessions on {8, 32}: 32 + 1 (size 8), not two half groups
    g, b = qt.qt_sched_plan([2] * 33, [8, 32])
    assert b == [32, 8] and g.count(0) == 32


@pytest.mark.parametrize("buckets", [[], [0], [4, 4], [8, 4], [33], list(range(1, 10))])
def test_plan_rejects_bad_buckets(qt, buckets):
    with pytest.raises(qt.QtError) as e:
        qt.qt_sched_plan([0, 0], buckets)
    assert e.value.status == 1


def test_plan_rejects_negative_class(qt):
    with pytest.raises(qt.QtError) as e:
        qt.qt_sched_plan([0, -1], [4])
    assert e.value.status == 1


def _scfg(qt, **over):
    kw = dict(buckets=[1, 2, 4, 8, 16, 32], max_sessions=64, max_pages=136, eos_index=2150)
    kw.update(over)
    return qt.make_sched_cfg(**kw)


def test_sched_bytes(qt):
    cfg = qt.make_cfg(synth.FULL)
    dev, host = qt.qt_sched_bytes(cfg, _scfg(qt))
    ws = qt.qt_workspace_bytes(cfg, 32, 136)
    d = synth.FULL
    per_session = (d.talker_vocab + d.n_steps * d.code_vocab + d.n_codebooks + 1) * 4 + 136 * 4
    assert dev >= ws + 64 * per_session
    assert dev % 256 == 0
    assert host >= 64 * 4 + 64 * 136 * 4
    dev2, host2 = qt.qt_sched_bytes(cfg, _scfg(qt, max_sessions=128))
    assert dev2 > dev and host2 > host
    # only the largest bucket sizes the shared batch tables
    dev3, _ = qt.qt_sched_bytes(cfg, _scfg(qt, buckets=[32]))
    assert dev3 == dev


@pytest.mark.parametrize("over", [
    dict(buckets=[]), dict(buckets=[2, 2]), dict(buckets=[64]), dict(buckets=list(range(1, 10))),
    dict(max_sessions=0), dict(max_sessions=5000), dict(max_pages=0), dict(eos_index=-2),
    dict(eos_index=3072),
])
def test_sched_cfg_rejected(qt, over):
    cfg = qt.make_cfg(synth.FULL)
    with pytest.raises(qt.QtError) as e:
        qt.qt_sched_bytes(cfg, _scfg(qt, **over))
    assert e.value.status == 1


def test_sched_calls_reject_null_handles(qt):
    import ctypes as C
    L = qt.lib()
    i32 = C.c_int32()
    p = C.c_void_p()
    assert L.qt_sched_open(None, 0, 1, 1, None, C.byref(i32)) == 1
    assert L.qt_sched_submit(None, 0, None, None) == 1
    assert L.qt_sched_step(None, None) == 1
    assert L.qt_sched_state(None, 0, C.byref(i32), None) == 1
    assert L.qt_sched_length(None, 0, C.byref(i32)) == 1
    assert L.qt_sched_free_pages(None, C.byref(i32)) == 1
    assert L.qt_sched_close(None, 0) == 1
    assert L.qt_sched_status_word(None, C.byref(p)) == 1
    assert L.qt_sched_outputs(None, 0, None, None, None, None) == 1
    kv = qt.KvCaches(None, None, 4)
    assert L.qt_sched_create(None, C.byref(_scfg(qt)), C.byref(kv), None, 0, None, 0, None,
                             C.byref(p)) == 1
    assert p.value is None
    L.qt_sched_destroy(None)
