"""Host-only checks of the C-ABI library (no GPU needed): it loads, exports
every function the headers under include/ declare, and rejects invalid arguments with the
documented status codes before anything reaches the device."""
import ctypes as C
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qt.h")
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def qt():
    import streaming_tts_decode_amd as qt
    qt.lib()
    return qt


def header_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qt_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function(qt):
    names = header_functions()
    assert len(names) >= 31
    lib = C.CDLL(qt.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"libqt.so does not export {n}"
    assert sorted(qt.EXPORTED) == names


def test_abi_version_matches_header(qt):
    v = int(re.search(r"#define QT_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert qt.qt_abi_version() == v


def _cfg(qt, dims=synth.FULL, **over):
    c = qt.make_cfg(dims)
    for k, v in over.items():
        if "." in k:
            a, b = k.split(".")
            setattr(getattr(c, a), b, v)
        else:
            setattr(c, k, v)
    return c


@pytest.mark.parametrize("over", [
    {"talker.head_dim": 64}, {"predictor.n_q_heads": 12}, {"talker.hidden": 1000},
    {"talker.ffn": 100}, {"page_size": 32}, {"n_codebooks": 17}, {"n_codebooks": 1},
    {"cb0_range": 0}, {"code_vocab": 100}, {"talker.layers": 0}, {"talker.rms_eps": 0.0},
])
def test_invalid_configs_are_rejected(qt, over):
    with pytest.raises(qt.QtError) as e:
        qt.qt_validate_cfg(_cfg(qt, **over))
    assert e.value.status == 2
    assert qt.qt_last_error()


def test_valid_configs(qt):
    for d in (synth.FULL, synth.SMALL):
        qt.qt_validate_cfg(_cfg(qt, d))
    assert qt.lib().qt_validate_cfg(None) == 1


def test_packed_bytes(qt):
    c = _cfg(qt)
    specs = synth.tensor_specs(synth.FULL)
    raw = sum(2 * int(__import__("numpy").prod(s)) for _, s, _ in specs)
    bf = qt.qt_packed_bytes(c, 0)
    assert raw <= bf <= raw + 256 * len(specs)
    i8 = qt.qt_packed_bytes(c, 1)
    # INT8 mode: one byte per Talker / head / projection weight plus its half copy
    # for the prompt prefill, the code predictor's quantized values as halves (two
    # bytes), f32 scales for every weight row
    w8 = sum(int(__import__("numpy").prod(s)) for n, s, k in specs
             if k == synth.WEIGHT and not n.startswith("predictor."))
    rows = sum(s[0] for _, s, k in specs if k == synth.WEIGHT)
    assert raw + w8 + 4 * rows <= i8 <= raw + w8 + 4 * rows + 768 * len(specs)
    with pytest.raises(qt.QtError):
        qt.qt_packed_bytes(c, 2)


def test_workspace_bytes(qt):
    c = _cfg(qt)
    a = qt.qt_workspace_bytes(c, 1, 10)
    b = qt.qt_workspace_bytes(c, 32, 10)
    d = qt.qt_workspace_bytes(c, 32, 200)
    assert 0 < a < b < d
    with pytest.raises(qt.QtError) as e:
        qt.qt_workspace_bytes(c, 33, 10)
    assert e.value.status == 9
    with pytest.raises(qt.QtError) as e:
        qt.qt_workspace_bytes(c, 0, 10)
    assert e.value.status == 1


def _table(dims, ptr=0x10000):
    out = []
    for name, shape, _ in synth.tensor_specs(dims):
        rows, cols = (1, shape[0]) if len(shape) == 1 else shape
        out.append([name, ptr, 0, rows, cols])
    return out


def _load(qt, table, dims=synth.SMALL, packed=0x100000, nbytes=None, int8=0):
    c = _cfg(qt, dims)
    if nbytes is None:
        nbytes = qt.qt_packed_bytes(c, int8)
    with pytest.raises(qt.QtError) as e:
        qt.qt_load_weights(c, [tuple(t) for t in table], int8, packed, nbytes)
    return e.value.status


def test_load_weights_checks_coverage_both_ways(qt):
    t = _table(synth.SMALL)
    assert _load(qt, t[1:]) == 4                                  # missing
    assert _load(qt, t + [["talker.extra", 0x10000, 0, 1, 8]]) == 5  # unexpected
    assert _load(qt, t + [t[3]]) == 5                             # duplicated
    bad = [list(x) for x in t]
    bad[2][4] += 1
    assert _load(qt, bad) == 2                                    # shape
    bad = [list(x) for x in t]
    bad[5][2] = 1
    assert _load(qt, bad) == 3                                    # dtype
    bad = [list(x) for x in t]
    bad[0][1] = 0
    assert _load(qt, bad) == 1                                    # no data
    assert _load(qt, t, packed=0) == 1                            # no packed buffer
    assert _load(qt, t, packed=0x100010) == 1                     # misaligned
    assert _load(qt, t, nbytes=1024) == 6                         # too small


def test_frame_and_quantize_argument_errors(qt):
    lib = qt.lib()
    assert lib.qt_frame_decode(None, None, None, None, None, None, 0, None) == 1
    assert lib.qt_quantize_int8(None, 4, 4, None, None, None) == 1
    assert lib.qt_quantize_int8(C.c_void_p(16), 0, 4, C.c_void_p(16), C.c_void_p(16), None) == 1
    g = C.c_void_p()
    assert lib.qt_frame_graph_create(None, None, None, None, None, None, 0, C.byref(g)) == 1
    assert lib.qt_frame_graph_launch(None, None) == 1
    lib.qt_graph_destroy(None)
    lib.qt_model_destroy(None)


def test_frame_launch_count(qt):
    """Launches per frame: entry + exit + the head GEMM; 5 per Talker layer (QKV,
    attention, o, gate/up, down), 6 from 16 sessions on (the attention's split merge
    in a launch of its own); per predictor step a gather, 5 per layer, a head."""
    for dims in (synth.FULL, synth.SMALL):
        c = qt.make_cfg(dims)
        t, p, steps = dims.talker.layers, dims.predictor.layers, dims.n_codebooks - 1
        for B in (1, 15, 16, 32):
            per = 6 if B >= 16 else 5
            assert qt.qt_frame_launch_count(c, qt.MODE_FULL, B) == 3 + per * t + steps * (2 + 5 * p)
            assert qt.qt_frame_launch_count(c, qt.MODE_TALKER, B) == 3 + per * t
            assert qt.qt_frame_launch_count(c, qt.MODE_PREDICTOR, B) == 3 + steps * (2 + 5 * p)
    assert qt.qt_frame_launch_count(qt.make_cfg(synth.FULL), qt.MODE_FULL, 1) == 548
    assert qt.qt_frame_launch_count(qt.make_cfg(synth.FULL), qt.MODE_FULL, 32) == 576
    for mode, B in ((7, 1), (qt.MODE_FULL, 0), (qt.MODE_FULL, 33)):
        with pytest.raises(qt.QtError) as e:
            qt.qt_frame_launch_count(qt.make_cfg(synth.FULL), mode, B)
        assert e.value.status == 1


def test_trace_argument_errors(qt):
    lib = qt.lib()
    t = C.c_void_p()
    assert lib.qt_trace_create(0, C.byref(t)) == 1
    assert lib.qt_trace_create(-5, C.byref(t)) == 1
    assert lib.qt_trace_create(10, None) == 1
    assert lib.qt_frame_trace(None, None, None, None, None, None, 0, None, None) == 1
    n = C.c_int32()
    assert lib.qt_trace_read(None, None, None, 0, C.byref(n)) == 1
    lib.qt_trace_destroy(None)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    import streaming_tts_decode_amd as qt
    monkeypatch.setattr(qt, "_lib", None)
    monkeypatch.setattr(qt, "LIB_PATH", str(tmp_path / "libqt.so"))
    with pytest.raises(RuntimeError):
        qt.lib()


def test_prefill_workspace_and_argument_errors(qt):
    import ctypes as C
    cfg = qt.make_cfg(synth.FULL)
    small = qt.qt_prefill_workspace_bytes(cfg, 64, 1)
    big = qt.qt_prefill_workspace_bytes(cfg, 1024, 4)
    assert small > 0 and big > 8 * small
    assert qt.qt_prefill_workspace_bytes(cfg, 1024, 32) > big
    # rows: multiples of 16, of 64 above 64, at most QT_PREFILL_MAX_ROWS
    for rows in (0, 8, 40, 80, 4096 + 64):
        with pytest.raises(qt.QtError) as e:
            qt.qt_prefill_workspace_bytes(cfg, rows, 1)
        assert e.value.status == 2, rows
    for seqs in (0, 33):
        with pytest.raises(qt.QtError) as e:
            qt.qt_prefill_workspace_bytes(cfg, 64, seqs)
        assert e.value.status == 1
    L = qt.lib()
    args = qt.PrefillArgs(64, 1, None, None, None, 4, None, None, None, None, None)
    kv = qt.KvCaches(None, None, 4)
    assert L.qt_prefill(None, C.byref(args), C.byref(kv), None, 0, None) == 1
    g = C.c_void_p()
    assert L.qt_prefill_graph_create(None, C.byref(args), C.byref(kv), None, 0, C.byref(g)) == 1
    assert g.value is None


def test_sampling_descriptor_layout(qt):
    """The ctypes mirror of qt_sampler_params / qt_sampling / qt_frame_inputs matches
    the C layout the header declares (16-byte parameters, four pointers, the
    sampling pointer last in the inputs)."""
    import ctypes as C
    assert C.sizeof(qt.SamplerParams) == 16
    assert C.sizeof(qt.Sampling) == 32
    assert qt.FrameInputs.sampling.offset == 40 and C.sizeof(qt.FrameInputs) == 48
    assert C.sizeof(qt.PrefillArgs) == 80
