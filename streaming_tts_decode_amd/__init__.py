"""Python binding of libqt.so, the gfx950 lockstep decode-frame library.

The functions below carry the C ABI's names (see include/qt.h) and only
marshal arguments: every step of the frame runs in the library's HIP kernels.
Importing this package never falls back to anything else: if libqt.so is
missing or cannot be loaded, `lib()` raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqt.so")

QT_OK = 0
STATUS_NAMES = {0: "QT_OK", 1: "QT_E_INVALID_ARG", 2: "QT_E_SHAPE", 3: "QT_E_DTYPE",
                4: "QT_E_MISSING_TENSOR", 5: "QT_E_UNEXPECTED_TENSOR", 6: "QT_E_CAPACITY",
                7: "QT_E_STATE", 8: "QT_E_HIP", 9: "QT_E_UNSUPPORTED"}
QT_BF16, QT_F32, QT_I8, QT_I32 = 0, 1, 2, 3
MODE_FULL, MODE_TALKER, MODE_PREDICTOR = 0, 1, 2
MODES = {"full": MODE_FULL, "talker": MODE_TALKER, "predictor": MODE_PREDICTOR}
STATUS_KV_OVERFLOW, STATUS_BAD_PAGE, STATUS_BAD_TOKEN, STATUS_NAN = 1, 2, 4, 8
STATUS_BAD_SAMPLER = 16
STATUS_FP16_RANGE = 32
STATUS_SYNC = 64
NOALLOC_SCRATCH_BYTES = 48 << 20
SAMPLER_MAX_TOP_K = 64

EXPORTED = ["qt_last_error", "qt_abi_version", "qt_validate_cfg", "qt_packed_bytes",
            "qt_workspace_bytes", "qt_load_weights", "qt_quantize_int8", "qt_model_export_int8",
            "qt_frame_decode", "qt_frame_decode_noalloc", "qt_frame_graph_create",
            "qt_frame_graph_launch",
            "qt_graph_destroy", "qt_model_destroy", "qt_trace_create", "qt_frame_launch_count",
            "qt_frame_trace", "qt_trace_read", "qt_trace_destroy",
            "qt_prefill_workspace_bytes", "qt_prefill", "qt_prefill_graph_create", "qt_sample",
            # qt_sched.h
            "qt_sched_bytes", "qt_sched_create", "qt_sched_open", "qt_sched_submit",
            "qt_sched_step", "qt_sched_outputs", "qt_sched_state", "qt_sched_length",
            "qt_sched_status_word", "qt_sched_free_pages", "qt_sched_close", "qt_sched_plan",
            "qt_sched_destroy", "qt_sched_set_sampling"]
SCHED_MAX_BUCKETS, SCHED_MAX_BATCH, SCHED_MAX_SESSIONS = 8, 32, 4096
SESSION_FREE, SESSION_RUNNING, SESSION_ENDED_EOS, SESSION_ENDED_MAX = 0, 1, 2, 3
KERNEL_KINDS = {0: "frame_begin", 1: "gemm", 2: "attn_paged", 3: "attn_pred", 4: "embed",
                5: "frame_end", 6: "predictor", 7: "attn_merge"}


class QtError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class DecoderCfg(C.Structure):
    _fields_ = [("layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("rope_theta", C.c_float), ("rms_eps", C.c_float)]


class ModelCfg(C.Structure):
    _fields_ = [("talker", DecoderCfg), ("predictor", DecoderCfg), ("talker_vocab", C.c_int32),
                ("code_vocab", C.c_int32), ("cb0_range", C.c_int32), ("n_codebooks", C.c_int32),
                ("page_size", C.c_int32)]


class Tensor(C.Structure):
    _fields_ = [("name", C.c_char_p), ("data", C.c_void_p), ("dtype", C.c_int32),
                ("rows", C.c_int64), ("cols", C.c_int64)]


class Sessions(C.Structure):
    _fields_ = [("batch", C.c_int32), ("kv_len", C.c_void_p), ("page_table", C.c_void_p),
                ("max_pages", C.c_int32)]


class KvCaches(C.Structure):
    _fields_ = [("k_pages", C.c_void_p), ("v_pages", C.c_void_p), ("num_pages", C.c_int32)]


class SamplerParams(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_p", C.c_float),
                ("repetition_penalty", C.c_float), ("top_k", C.c_int32)]


class Sampling(C.Structure):
    _fields_ = [("params", C.c_void_p), ("seed", C.c_void_p), ("counter", C.c_void_p),
                ("seen0", C.c_void_p)]


class FrameInputs(C.Structure):
    _fields_ = [("mode", C.c_int32), ("talker_in", C.c_void_p), ("h_in", C.c_void_p),
                ("tok0_in", C.c_void_p), ("forced", C.c_void_p),
                ("sampling", C.POINTER(Sampling))]


class FrameOutputs(C.Structure):
    _fields_ = [("logits0", C.c_void_p), ("logits_pred", C.c_void_p), ("tokens", C.c_void_p),
                ("status", C.c_void_p)]


class PrefillArgs(C.Structure):
    _fields_ = [("rows", C.c_int32), ("max_seqs", C.c_int32), ("seq_start", C.c_void_p),
                ("embeds", C.c_void_p), ("page_table", C.c_void_p), ("max_pages", C.c_int32),
                ("kv_len", C.c_void_p), ("logits0", C.c_void_p), ("tok0", C.c_void_p),
                ("h_last", C.c_void_p), ("status", C.c_void_p)]


PREFILL_MAX_SEQS, PREFILL_MAX_ROWS = 32, 4096


class LaunchInfo(C.Structure):
    _fields_ = [("kind", C.c_int32), ("step", C.c_int32), ("layer", C.c_int32), ("m", C.c_int32),
                ("n", C.c_int32), ("k", C.c_int32), ("int8", C.c_int32), ("n_logits", C.c_int32),
                ("name", C.c_char * 40)]


class SchedCfg(C.Structure):
    _fields_ = [("n_buckets", C.c_int32), ("buckets", C.c_int32 * SCHED_MAX_BUCKETS),
                ("max_sessions", C.c_int32), ("max_pages", C.c_int32), ("eos_index", C.c_int32)]


def make_sched_cfg(buckets, max_sessions: int, max_pages: int, eos_index: int = -1) -> SchedCfg:
    """n_buckets is len(buckets) even beyond SCHED_MAX_BUCKETS, which the library rejects."""
    buckets = list(buckets)
    kept = buckets[:SCHED_MAX_BUCKETS]
    arr = (C.c_int32 * SCHED_MAX_BUCKETS)(*(kept + [0] * (SCHED_MAX_BUCKETS - len(kept))))
    return SchedCfg(len(buckets), arr, max_sessions, max_pages, eos_index)


_lib = None
_P = C.c_void_p


def lib():
    """Load libqt.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m streaming_tts_decode_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        st = C.c_int
        L.qt_last_error.restype = C.c_char_p
        L.qt_last_error.argtypes = []
        L.qt_abi_version.restype = C.c_int32
        L.qt_validate_cfg.restype = st
        L.qt_validate_cfg.argtypes = [C.POINTER(ModelCfg)]
        L.qt_packed_bytes.restype = st
        L.qt_packed_bytes.argtypes = [C.POINTER(ModelCfg), C.c_int32, C.POINTER(C.c_uint64)]
        L.qt_workspace_bytes.restype = st
        L.qt_workspace_bytes.argtypes = [C.POINTER(ModelCfg), C.c_int32, C.c_int32,
                                         C.POINTER(C.c_uint64)]
        L.qt_load_weights.restype = st
        L.qt_load_weights.argtypes = [C.POINTER(ModelCfg), C.POINTER(Tensor), C.c_int32, C.c_int32,
                                      _P, C.c_uint64, _P, C.POINTER(_P)]
        L.qt_quantize_int8.restype = st
        L.qt_quantize_int8.argtypes = [_P, C.c_int64, C.c_int64, _P, _P, _P]
        L.qt_model_export_int8.restype = st
        L.qt_model_export_int8.argtypes = [_P, C.c_char_p, _P, _P, _P]
        frame_args = [_P, C.POINTER(Sessions), C.POINTER(KvCaches), C.POINTER(FrameInputs),
                      C.POINTER(FrameOutputs), _P, C.c_uint64]
        L.qt_frame_decode.restype = st
        L.qt_frame_decode.argtypes = frame_args + [_P]
        L.qt_frame_decode_noalloc.restype = st
        L.qt_frame_decode_noalloc.argtypes = frame_args[:5] + [_P]
        L.qt_frame_graph_create.restype = st
        L.qt_frame_graph_create.argtypes = frame_args + [C.POINTER(_P)]
        L.qt_frame_graph_launch.restype = st
        L.qt_frame_graph_launch.argtypes = [_P, _P]
        L.qt_graph_destroy.restype = None
        L.qt_graph_destroy.argtypes = [_P]
        L.qt_model_destroy.restype = None
        L.qt_model_destroy.argtypes = [_P]
        L.qt_trace_create.restype = st
        L.qt_trace_create.argtypes = [C.c_int32, C.POINTER(_P)]
        L.qt_frame_launch_count.restype = st
        L.qt_frame_launch_count.argtypes = [C.POINTER(ModelCfg), C.c_int32, C.c_int32,
                                            C.POINTER(C.c_int32)]
        L.qt_frame_trace.restype = st
        L.qt_frame_trace.argtypes = frame_args + [_P, _P]
        L.qt_trace_read.restype = st
        L.qt_trace_read.argtypes = [_P, C.POINTER(LaunchInfo), C.POINTER(C.c_float), C.c_int32,
                                    C.POINTER(C.c_int32)]
        L.qt_trace_destroy.restype = None
        L.qt_trace_destroy.argtypes = [_P]
        L.qt_sample.restype = st
        L.qt_sample.argtypes = [_P, C.c_int32, C.c_int32, C.c_int32, _P, _P, _P, C.c_int32, _P, _P,
                                _P, _P]
        L.qt_prefill_workspace_bytes.restype = st
        L.qt_prefill_workspace_bytes.argtypes = [C.POINTER(ModelCfg), C.c_int32, C.c_int32,
                                                 C.POINTER(C.c_uint64)]
        L.qt_prefill.restype = st
        L.qt_prefill.argtypes = [_P, C.POINTER(PrefillArgs), C.POINTER(KvCaches), _P, C.c_uint64, _P]
        L.qt_prefill_graph_create.restype = st
        L.qt_prefill_graph_create.argtypes = [_P, C.POINTER(PrefillArgs), C.POINTER(KvCaches), _P,
                                              C.c_uint64, C.POINTER(_P)]
        i32p = C.POINTER(C.c_int32)
        L.qt_sched_bytes.restype = st
        L.qt_sched_bytes.argtypes = [C.POINTER(ModelCfg), C.POINTER(SchedCfg),
                                     C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)]
        L.qt_sched_create.restype = st
        L.qt_sched_create.argtypes = [_P, C.POINTER(SchedCfg), C.POINTER(KvCaches), _P, C.c_uint64,
                                      _P, C.c_uint64, _P, C.POINTER(_P)]
        L.qt_sched_open.restype = st
        L.qt_sched_open.argtypes = [_P, C.c_int32, C.c_int32, C.c_int32, i32p, i32p]
        L.qt_sched_set_sampling.restype = st
        L.qt_sched_set_sampling.argtypes = [_P, C.c_int32, C.POINTER(SamplerParams), C.c_uint64]
        L.qt_sched_submit.restype = st
        L.qt_sched_submit.argtypes = [_P, C.c_int32, _P, _P]
        L.qt_sched_step.restype = st
        L.qt_sched_step.argtypes = [_P, i32p]
        L.qt_sched_outputs.restype = st
        L.qt_sched_outputs.argtypes = [_P, C.c_int32, C.POINTER(_P), C.POINTER(_P), C.POINTER(_P),
                                       i32p]
        L.qt_sched_state.restype = st
        L.qt_sched_state.argtypes = [_P, C.c_int32, i32p, i32p]
        L.qt_sched_length.restype = st
        L.qt_sched_length.argtypes = [_P, C.c_int32, i32p]
        L.qt_sched_status_word.restype = st
        L.qt_sched_status_word.argtypes = [_P, C.POINTER(_P)]
        L.qt_sched_free_pages.restype = st
        L.qt_sched_free_pages.argtypes = [_P, i32p]
        L.qt_sched_close.restype = st
        L.qt_sched_close.argtypes = [_P, C.c_int32]
        L.qt_sched_plan.restype = st
        L.qt_sched_plan.argtypes = [i32p, C.c_int32, i32p, C.c_int32, i32p, i32p, i32p]
        L.qt_sched_destroy.restype = None
        L.qt_sched_destroy.argtypes = [_P]
        _lib = L
    return _lib


def _check(status: int, fn: str):
    if status != QT_OK:
        raise QtError(status, fn, lib().qt_last_error().decode())


def make_cfg(dims) -> ModelCfg:
    """qt_model_cfg from a dimension record with talker/predictor sub-records."""
    def dec(d):
        return DecoderCfg(d.layers, d.hidden, d.n_q, d.n_kv, d.head_dim, d.ffn,
                          float(d.rope_theta), float(d.eps))
    return ModelCfg(dec(dims.talker), dec(dims.predictor), dims.talker_vocab, dims.code_vocab,
                    dims.cb0_range, dims.n_codebooks, dims.page_size)


# --------------------------------------------------------------------------- ABI calls
def qt_last_error() -> str:
    return lib().qt_last_error().decode()


def qt_abi_version() -> int:
    return lib().qt_abi_version()


def qt_validate_cfg(cfg: ModelCfg) -> None:
    _check(lib().qt_validate_cfg(C.byref(cfg)), "qt_validate_cfg")


def qt_packed_bytes(cfg: ModelCfg, int8_mode: int) -> int:
    n = C.c_uint64()
    _check(lib().qt_packed_bytes(C.byref(cfg), int8_mode, C.byref(n)), "qt_packed_bytes")
    return n.value


def qt_workspace_bytes(cfg: ModelCfg, max_batch: int, max_pages: int) -> int:
    n = C.c_uint64()
    _check(lib().qt_workspace_bytes(C.byref(cfg), max_batch, max_pages, C.byref(n)),
           "qt_workspace_bytes")
    return n.value


def qt_load_weights(cfg: ModelCfg, tensors, int8_mode: int, packed_ptr: int, packed_bytes: int,
                    stream: int = 0) -> int:
    """tensors: iterable of (name, device_ptr, dtype, rows, cols).  Returns the model handle."""
    tensors = list(tensors)
    arr = (Tensor * len(tensors))()
    names = []
    for i, (name, ptr, dt, rows, cols) in enumerate(tensors):
        nb = name.encode()
        names.append(nb)
        arr[i] = Tensor(nb, ptr, dt, rows, cols)
    out = _P()
    _check(lib().qt_load_weights(C.byref(cfg), arr, len(tensors), int8_mode, packed_ptr,
                                 packed_bytes, stream, C.byref(out)), "qt_load_weights")
    return out.value


def qt_quantize_int8(w_ptr: int, rows: int, cols: int, q_ptr: int, scale_ptr: int,
                     stream: int = 0) -> None:
    _check(lib().qt_quantize_int8(w_ptr, rows, cols, q_ptr, scale_ptr, stream), "qt_quantize_int8")


def qt_model_export_int8(model: int, name: str, q_ptr: int, scale_ptr: int, stream: int = 0) -> None:
    _check(lib().qt_model_export_int8(model, name.encode(), q_ptr, scale_ptr, stream),
           "qt_model_export_int8")


def qt_frame_decode(model: int, sessions: Sessions, kv: KvCaches, inputs: FrameInputs,
                    outputs: FrameOutputs, workspace_ptr: int, workspace_bytes: int,
                    stream: int = 0) -> None:
    _check(lib().qt_frame_decode(model, C.byref(sessions), C.byref(kv), C.byref(inputs),
                                 C.byref(outputs), workspace_ptr, workspace_bytes, stream),
           "qt_frame_decode")


def qt_frame_decode_noalloc(model: int, sessions: Sessions, kv: KvCaches, inputs: FrameInputs,
                            outputs: FrameOutputs, stream: int = 0) -> None:
    """qt_frame_decode with the library's static scratch instead of a workspace."""
    _check(lib().qt_frame_decode_noalloc(model, C.byref(sessions), C.byref(kv), C.byref(inputs),
                                         C.byref(outputs), stream), "qt_frame_decode_noalloc")


def qt_frame_graph_create(model: int, sessions: Sessions, kv: KvCaches, inputs: FrameInputs,
                          outputs: FrameOutputs, workspace_ptr: int, workspace_bytes: int) -> int:
    g = _P()
    _check(lib().qt_frame_graph_create(model, C.byref(sessions), C.byref(kv), C.byref(inputs),
                                       C.byref(outputs), workspace_ptr, workspace_bytes,
                                       C.byref(g)), "qt_frame_graph_create")
    return g.value


def qt_frame_graph_launch(graph: int, stream: int = 0) -> None:
    _check(lib().qt_frame_graph_launch(graph, stream), "qt_frame_graph_launch")


def qt_graph_destroy(graph: int) -> None:
    lib().qt_graph_destroy(graph)


def qt_model_destroy(model: int) -> None:
    lib().qt_model_destroy(model)


def qt_trace_create(max_launches: int) -> int:
    t = _P()
    _check(lib().qt_trace_create(max_launches, C.byref(t)), "qt_trace_create")
    return t.value


def qt_frame_launch_count(cfg: ModelCfg, mode: int, batch: int) -> int:
    n = C.c_int32()
    _check(lib().qt_frame_launch_count(C.byref(cfg), mode, batch, C.byref(n)), "qt_frame_launch_count")
    return n.value


def qt_frame_trace(model: int, sessions: Sessions, kv: KvCaches, inputs: FrameInputs,
                   outputs: FrameOutputs, workspace_ptr: int, workspace_bytes: int, stream: int,
                   trace: int) -> None:
    _check(lib().qt_frame_trace(model, C.byref(sessions), C.byref(kv), C.byref(inputs),
                                C.byref(outputs), workspace_ptr, workspace_bytes, stream, trace),
           "qt_frame_trace")


def qt_trace_read(trace: int, max_launches: int):
    """[(LaunchInfo, milliseconds)] of the last traced frame (waits for it)."""
    info = (LaunchInfo * max_launches)()
    ms = (C.c_float * max_launches)()
    n = C.c_int32()
    _check(lib().qt_trace_read(trace, info, ms, max_launches, C.byref(n)), "qt_trace_read")
    return [(info[i], float(ms[i])) for i in range(n.value)]


def qt_trace_destroy(trace: int) -> None:
    lib().qt_trace_destroy(trace)


def qt_sample(logits_ptr: int, rows: int, ld: int, V: int, params_ptr: int, seed_ptr: int,
              counter_ptr: int, codebook: int, seen_ptr: int | None, tokens_ptr: int,
              status_ptr: int, stream: int = 0) -> None:
    _check(lib().qt_sample(logits_ptr, rows, ld, V, params_ptr, seed_ptr, counter_ptr, codebook,
                           seen_ptr, tokens_ptr, status_ptr, stream), "qt_sample")


def qt_prefill_workspace_bytes(cfg: ModelCfg, rows: int, max_seqs: int) -> int:
    n = C.c_uint64()
    _check(lib().qt_prefill_workspace_bytes(C.byref(cfg), rows, max_seqs, C.byref(n)),
           "qt_prefill_workspace_bytes")
    return n.value


def qt_prefill(model: int, args: PrefillArgs, kv: KvCaches, workspace_ptr: int, workspace_bytes: int,
               stream: int = 0) -> None:
    _check(lib().qt_prefill(model, C.byref(args), C.byref(kv), workspace_ptr, workspace_bytes, stream),
           "qt_prefill")


def qt_prefill_graph_create(model: int, args: PrefillArgs, kv: KvCaches, workspace_ptr: int,
                            workspace_bytes: int) -> int:
    g = _P()
    _check(lib().qt_prefill_graph_create(model, C.byref(args), C.byref(kv), workspace_ptr,
                                         workspace_bytes, C.byref(g)), "qt_prefill_graph_create")
    return g.value


# --------------------------------------------------------------------------- scheduler (qt_sched.h)
def qt_sched_bytes(cfg: ModelCfg, scfg: SchedCfg):
    """(device_bytes, host_bytes) the scheduler needs."""
    d, h = C.c_uint64(), C.c_uint64()
    _check(lib().qt_sched_bytes(C.byref(cfg), C.byref(scfg), C.byref(d), C.byref(h)),
           "qt_sched_bytes")
    return d.value, h.value


def qt_sched_create(model: int, scfg: SchedCfg, kv: KvCaches, device_ptr: int, device_bytes: int,
                    host_ptr: int, host_bytes: int, stream: int = 0) -> int:
    out = _P()
    _check(lib().qt_sched_create(model, C.byref(scfg), C.byref(kv), device_ptr, device_bytes,
                                 host_ptr, host_bytes, stream, C.byref(out)), "qt_sched_create")
    return out.value


def qt_sched_open(sched: int, length: int, min_frames: int, max_frames: int,
                  page_size: int = 16):
    """Returns (session id, list of the page ids that hold positions [0, length))."""
    n = -(-length // page_size) if length > 0 else 0
    pages = (C.c_int32 * max(n, 1))()
    sid = C.c_int32()
    _check(lib().qt_sched_open(sched, length, min_frames, max_frames, pages, C.byref(sid)),
           "qt_sched_open")
    return sid.value, list(pages)[:n]


def qt_sched_set_sampling(sched: int, session: int, params=None, seed: int = 0):
    """params: (codebook-0, predictor) pair of (temperature, top_p, repetition_penalty,
    top_k) tuples, or None for greedy tokens."""
    arr = None
    if params is not None:
        arr = (SamplerParams * 2)(*(SamplerParams(*p) for p in params))
    _check(lib().qt_sched_set_sampling(sched, session, arr, seed), "qt_sched_set_sampling")


def qt_sched_submit(sched: int, session: int, talker_in_ptr: int, forced_ptr: int | None = None):
    _check(lib().qt_sched_submit(sched, session, talker_in_ptr, forced_ptr), "qt_sched_submit")


def qt_sched_step(sched: int) -> int:
    ng = C.c_int32()
    _check(lib().qt_sched_step(sched, C.byref(ng)), "qt_sched_step")
    return ng.value


def qt_sched_outputs(sched: int, session: int):
    """(logits0_ptr, logits_pred_ptr, tokens_ptr, frames)."""
    a, b, c, f = _P(), _P(), _P(), C.c_int32()
    _check(lib().qt_sched_outputs(sched, session, C.byref(a), C.byref(b), C.byref(c), C.byref(f)),
           "qt_sched_outputs")
    return a.value, b.value, c.value, f.value


def qt_sched_state(sched: int, session: int):
    """(qt_session_state, end_frame)."""
    st, ef = C.c_int32(), C.c_int32()
    _check(lib().qt_sched_state(sched, session, C.byref(st), C.byref(ef)), "qt_sched_state")
    return st.value, ef.value


def qt_sched_length(sched: int, session: int) -> int:
    n = C.c_int32()
    _check(lib().qt_sched_length(sched, session, C.byref(n)), "qt_sched_length")
    return n.value


def qt_sched_status_word(sched: int) -> int:
    p = _P()
    _check(lib().qt_sched_status_word(sched, C.byref(p)), "qt_sched_status_word")
    return p.value


def qt_sched_free_pages(sched: int) -> int:
    n = C.c_int32()
    _check(lib().qt_sched_free_pages(sched, C.byref(n)), "qt_sched_free_pages")
    return n.value


def qt_sched_close(sched: int, session: int) -> None:
    _check(lib().qt_sched_close(sched, session), "qt_sched_close")


def qt_sched_plan(cls, buckets):
    """(group_of list, group_bucket list) for ready sessions of classes `cls`."""
    cls = list(cls)
    buckets = list(buckets)
    n = len(cls)
    c_cls = (C.c_int32 * max(n, 1))(*cls)
    c_b = (C.c_int32 * max(len(buckets), 1))(*buckets)
    g_of = (C.c_int32 * max(n, 1))()
    g_b = (C.c_int32 * max(n, 1))()
    ng = C.c_int32()
    _check(lib().qt_sched_plan(c_cls, n, c_b, len(buckets), g_of, g_b, C.byref(ng)), "qt_sched_plan")
    return list(g_of)[:n], list(g_b)[:ng.value]


def qt_sched_destroy(sched: int) -> None:
    lib().qt_sched_destroy(sched)
