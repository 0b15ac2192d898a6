"""GPU tests on the reduced model and the INT8 quantizer: batch sizes across the
VALU (M <= 2) and MFMA (M >= 3, with the activation-row split) GEMM forms, ragged
and boundary KV lengths, long contexts at full batch,
determinism, graph replay, paging invariance, device status bits, and the
bit-exact INT8 quantizer on every decode weight of the full model."""
import numpy as np
import pytest

import synth
from tests.gpu_cases import log, run_frames
from tests.parity import compare

pytestmark = pytest.mark.gpu

S = synth.SMALL


def small_w(name, mode="full", batch=1, frames=2, lens=(), lo=0, hi=0, **kw):
    return synth.Workload(name, mode, batch=batch, frames=frames, len_lo=lo, len_hi=hi,
                          dims=S, lens=tuple(lens), **kw)


# ----------------------------------------------------------------- batch sizes / paths
@pytest.mark.parametrize("B", [1, 2, 3, 5, 8, 9, 16, 20, 32])
def test_small_batches_match_oracle(small_pm, orc_small, B):
    """B <= 4 keeps every GEMM on the VALU path (predictor step 1 has 2B rows);
    B >= 5 moves step 1 to MFMA, B >= 9 moves every GEMM to MFMA."""
    lens = [(37 * b + 5) % 90 for b in range(B)]
    w = small_w(f"S{B}", batch=B, frames=2, lens=lens)
    run_frames(small_pm, orc_small, w, check=range(B))


def test_small_boundary_lengths(small_pm, orc_small):
    """Empty caches and page-boundary lengths (the new token opens a page, fills
    its last slot, or lands in a fresh split)."""
    lens = [0, 1, 15, 16, 17, 31, 32, 127, 128, 129, 255, 256]
    w = small_w("Sedge", batch=len(lens), frames=3, lens=lens)
    run_frames(small_pm, orc_small, w, check=range(len(lens)))


def test_small_long_context_many_splits(small_pm, orc_small):
    """B=2 with ~1.5k positions: the split-KV partials and their merge."""
    w = small_w("Slong", batch=2, frames=2, lens=[1500, 700])
    run_frames(small_pm, orc_small, w, check=[0, 1])


@pytest.mark.parametrize("lo,hi", [(1900, 2000), (3600, 4000)])
def test_small_long_context_full_batch(small_pm, orc_small, lo, hi):
    """B=32 with 2k and 4k contexts: many sessions with 16+ attention splits each,
    all merged by their last block."""
    w = small_w(f"Sgrp{hi}", batch=32, frames=1, lo=lo, hi=hi)
    L = w.lengths()
    run_frames(small_pm, orc_small, w, check=[int(np.argmax(L)), int(np.argmin(L))])


# ----------------------------------------------------------------- split merge in its own launch
# From 16 sessions on, the Talker attention's split partials are merged by a launch
# of their own (k_attn_merge) instead of by the last split to finish.
def test_sep_merge_boundary_lengths(small_pm, orc_small):
    """Empty caches and page-boundary lengths at B=16: one-split sessions (written
    by the split itself) beside sessions merged by the merge launch."""
    lens = [0, 1, 15, 16, 17, 31, 32, 127, 128, 129, 255, 256, 2, 47, 64, 300]
    w = small_w("Ssep_edge", batch=len(lens), frames=3, lens=lens)
    run_frames(small_pm, orc_small, w, check=range(len(lens)))


def test_sep_merge_short_sessions(small_pm, orc_small):
    """20 sessions of at most 3 pages: nearly every session has one split, which the
    merge launch leaves alone."""
    lens = [(7 * b) % 40 for b in range(20)]
    w = small_w("Ssep_short", batch=len(lens), frames=2, lens=lens)
    run_frames(small_pm, orc_small, w, check=range(len(lens)))


def test_sep_merge_long_and_short(small_pm, orc_small):
    """24 one-page sessions beside 8 of ~4k positions (32 splits each: two merge
    rounds of 16 partials)."""
    lens = [5] * 24 + [4090, 4000, 4095, 4050, 4080, 4020, 4060, 4010]
    w = small_w("Ssep_mix", batch=len(lens), frames=1, lens=lens)
    run_frames(small_pm, orc_small, w, check=[0, 3, 4, 7, 8, 15, 23, 24])


def test_small_graph_replay(small_pm, orc_small):
    w = small_w("Sgraph", batch=6, frames=4, lens=[3, 40, 77, 16, 130, 0], graph=True)
    run_frames(small_pm, orc_small, w, check=range(6), use_graph=True)


@pytest.mark.parametrize("mode", ["talker", "predictor"])
def test_small_modes(small_pm, orc_small, mode):
    w = small_w(f"Smode{mode}", mode=mode, batch=3, frames=2, lens=[5, 20, 33])
    run_frames(small_pm, orc_small, w, check=range(3))


# ----------------------------------------------------------------- invariances
def _run_eager(dec, w, frames_inputs, forced, use_graph=False, mode="full", traces=None):
    torch = dec.torch
    g = dec.capture(mode, forced=True) if use_graph else None
    outs = []
    for f in range(w.frames):
        dec.set_inputs(talker_in=frames_inputs["talker_in"][f], forced=forced[f])
        if g is not None:
            dec.replay(g)
        elif traces is not None:
            traces.append(dec.trace(mode, forced=True))
        else:
            dec.decode(mode, forced=True)
        torch.cuda.synchronize()
        outs.append((dec.logits0.cpu().numpy().copy(), dec.logits_pred.cpu().numpy().copy(),
                     dec.tokens.cpu().numpy().copy()))
    return outs


def _fresh(small_pm, w, page_seed=1234):
    from streaming_tts_decode_amd.runtime import Decoder
    t = S.talker
    dec = Decoder(small_pm, batch=w.batch, max_pages=w.max_pages(), page_seed=page_seed)
    for b, L in enumerate(w.lengths()):
        kb, vb = synth.gen_kv(w.name, b, t.layers, int(L), t.n_kv, t.head_dim)
        dec.load_session_kv(b, kb, vb)
    return dec


def _forced(w):
    rng = np.random.default_rng(5)
    return rng.integers(0, S.cb0_range, size=(w.frames, w.batch, S.n_codebooks)).astype(np.int32)


@pytest.mark.parametrize("B", [4, 20])
def test_replays_are_bitwise_deterministic_and_equal_eager(small_pm, B):
    """B=4: splits merged by the last to finish; B=20: merged by their own launch."""
    lens = [600, 5, 333, 48] if B == 4 else [(211 * b + 40) % 900 for b in range(B)]
    w = small_w(f"Sdet{B}", batch=B, frames=3, lens=lens)
    fi, fz = synth.frame_inputs(w), _forced(w)
    runs = []
    for use_graph in (False, False, True, True):
        dec = _fresh(small_pm, w)
        runs.append(_run_eager(dec, w, fi, fz, use_graph=use_graph))
        dec.close()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            for x, y in zip(a, b):
                np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("mode,B", [("full", 3), ("predictor", 3), ("full", 16)])
def test_traced_frame_equals_untraced(small_pm, mode, B):
    """qt_frame_trace runs the same kernels as qt_frame_decode: identical outputs,
    one timed interval per launch, and launch records that match the frame's structure
    (from 16 sessions on, a split-merge launch after each Talker attention)."""
    import streaming_tts_decode_amd as qt
    w = small_w(f"Strace{B}", batch=B, frames=2, lens=[[40, 300, 7][b % 3] + b for b in range(B)])
    fi, fz = synth.frame_inputs(w), _forced(w)
    plain = _run_eager(_fresh(small_pm, w), w, fi, fz, mode=mode)
    traces = []
    dec = _fresh(small_pm, w)
    traced = _run_eager(dec, w, fi, fz, mode=mode, traces=traces)
    dec.close()
    for a, b in zip(plain, traced):
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
    t, p = S.talker, S.predictor
    n_steps = S.n_codebooks - 1
    for rec in traces:
        assert len(rec) == qt.qt_frame_launch_count(small_pm.cfg, qt.MODES[mode], B)
        assert rec[0][1] == "frame_begin" and rec[-1][1] == "frame_end"
        assert all(ms > 0 for *_, ms in rec)
        kinds = [k for _, k, _, _ in rec]
        gemms = [li for _, k, li, _ in rec if k == "gemm"]
        n_tl = t.layers if mode == "full" else 0
        assert kinds.count("attn_paged") == n_tl
        assert kinds.count("attn_merge") == (n_tl if B >= 16 else 0)
        for i, k in enumerate(kinds):  # a merge follows its attention launch
            if k == "attn_merge":
                assert kinds[i - 1] == "attn_paged"
        assert kinds.count("attn_pred") == n_steps * p.layers
        assert kinds.count("embed") == n_steps
        assert len(gemms) == 4 * n_tl + 1 + n_steps * (4 * p.layers + 1)
        for name, kind, li, _ in rec:
            assert name.startswith("k_" + ("gemm" if kind == "gemm" else kind))
        # one QKV GEMM per layer with the fused [q; k; v] shape, rows = sessions
        # (predictor step 1 carries two positions per session)
        qkv_n = lambda d: (d.n_q + 2 * d.n_kv) * d.head_dim
        for li in gemms:
            if li.n == qkv_n(t) and li.k == t.hidden and li.step == 0:
                assert li.m == w.batch
            if li.n == qkv_n(p) and li.k == p.hidden:
                assert li.m == (2 if li.step == 1 else 1) * w.batch
        heads = [li for li in gemms if li.n_logits]
        assert len(heads) == (1 if mode == "full" else 0) + n_steps
        assert all(li.n_logits == S.code_vocab for li in heads if li.step > 0)


@pytest.mark.parametrize("B", [3, 18])
def test_page_permutation_invariance(small_pm, B):
    lens = [200, 17, 90] if B == 3 else [(97 * b + 17) % 500 for b in range(B)]
    w = small_w(f"Sperm{B}", batch=B, frames=2, lens=lens)
    fi, fz = synth.frame_inputs(w), _forced(w)
    a = _run_eager(_fresh(small_pm, w, page_seed=1), w, fi, fz)
    b = _run_eager(_fresh(small_pm, w, page_seed=2), w, fi, fz)
    for x, y in zip(a, b):
        for u, v in zip(x, y):
            np.testing.assert_array_equal(u, v)


def test_lockstep_batch_equals_single_sessions(small_pm):
    w = small_w("Slock", batch=6, frames=2, lens=[10, 50, 90, 130, 170, 210])
    fi, fz = synth.frame_inputs(w), _forced(w)
    batch = _run_eager(_fresh(small_pm, w), w, fi, fz)
    lens = w.lengths()
    for b in range(w.batch):
        w1 = small_w("Slock", batch=1, frames=2, lens=[int(lens[b])])
        dec = _fresh(small_pm, w1)
        t = S.talker
        kb, vb = synth.gen_kv("Slock", b, t.layers, int(lens[b]), t.n_kv, t.head_dim)
        dec.load_session_kv(0, kb, vb)
        single = _run_eager(dec, w1, {"talker_in": fi["talker_in"][:, b:b + 1]}, fz[:, b:b + 1])
        for f in range(w.frames):
            compare(single[f][0][0], batch[f][0][b], S.cb0_range, label=f"lockstep s{b} f{f} cb0")
            compare(single[f][1][0], batch[f][1][b], label=f"lockstep s{b} f{f} pred")


def test_talker_mode_equals_full_mode_codebook0(small_pm):
    w = small_w("Stm", batch=3, frames=1, lens=[9, 99, 199])
    fi, fz = synth.frame_inputs(w), _forced(w)
    full = _run_eager(_fresh(small_pm, w), w, fi, fz, mode="full")
    talk = _run_eager(_fresh(small_pm, w), w, fi, fz, mode="talker")
    np.testing.assert_array_equal(full[0][0], talk[0][0])
    np.testing.assert_array_equal(full[0][2][:, 0], talk[0][2][:, 0])


# ----------------------------------------------------------------- device status
@pytest.mark.parametrize("B", [2, 16])
def test_capacity_overflow_is_flagged_and_skipped(small_pm, orc_small, B):
    from streaming_tts_decode_amd import STATUS_KV_OVERFLOW
    w = small_w(f"Sover{B}", batch=B, frames=1, lens=[20, 30] + [9] * (B - 2))
    dec = _fresh(small_pm, w)
    cap = dec.max_pages * 16
    dec.kv_len[1] = cap  # session 1 is full
    fi = synth.frame_inputs(w)
    dec.set_inputs(talker_in=fi["talker_in"][0])
    dec.status.zero_()
    dec.decode("full")
    dec.torch.cuda.synchronize()
    st = int(dec.status.item())
    assert st & STATUS_KV_OVERFLOW
    kv = dec.kv_len.cpu().numpy()
    assert kv[1] == cap and kv[0] == 21
    # session 0 is still decoded correctly
    t = S.talker
    kb, vb = synth.gen_kv(f"Sover{B}", 0, t.layers, 20, t.n_kv, t.head_dim)
    o = orc_small.run_session("talker", 1, talker_in=fi["talker_in"][:, 0], k_bits=kb, v_bits=vb,
                              length=20)
    compare(dec.logits0.cpu().numpy()[0:1], o["logits0"], S.cb0_range, label="overflow s0")


@pytest.mark.parametrize("B", [2, 16])
def test_bad_page_and_bad_token_are_flagged(small_pm, B):
    from streaming_tts_decode_amd import STATUS_BAD_PAGE, STATUS_BAD_TOKEN
    w = small_w(f"Sbad{B}", batch=B, frames=1, lens=[40] * B)
    dec = _fresh(small_pm, w)
    fi = synth.frame_inputs(w)
    pt = dec.page_table.cpu().numpy()
    pt[0, 1] = dec.num_pages + 7  # out of range, read as zeros
    dec.page_table.copy_(dec.torch.from_numpy(pt))
    forced = np.zeros((B, S.n_codebooks), dtype=np.int32)
    forced[1, 2] = S.code_vocab + 3  # out of range
    dec.set_inputs(talker_in=fi["talker_in"][0], forced=forced)
    dec.status.zero_()
    dec.decode("full", forced=True)
    dec.torch.cuda.synchronize()
    st = int(dec.status.item())
    assert st & STATUS_BAD_PAGE and st & STATUS_BAD_TOKEN
    assert np.all(np.isfinite(dec.logits_pred.cpu().numpy()))


# ----------------------------------------------------------------- ABI errors needing a model
def test_frame_argument_errors(small_pm):
    import streaming_tts_decode_amd as qt
    from streaming_tts_decode_amd.runtime import Decoder
    dec = Decoder(small_pm, batch=2, max_pages=4)
    ss, kv, fi, fo = dec._descs("full", False)
    with pytest.raises(qt.QtError) as e:
        qt.qt_frame_decode(dec.model, ss, kv, fi, fo, dec.ws_ptr, 1024)
    assert e.value.status == 6  # QT_E_CAPACITY
    ss.batch = 33
    with pytest.raises(qt.QtError) as e:
        qt.qt_frame_decode(dec.model, ss, kv, fi, fo, dec.ws_ptr, dec.ws_bytes)
    assert e.value.status == 9  # QT_E_UNSUPPORTED
    ss.batch = 2
    fi.mode = 7
    with pytest.raises(qt.QtError) as e:
        qt.qt_frame_decode(dec.model, ss, kv, fi, fo, dec.ws_ptr, dec.ws_bytes)
    assert e.value.status == 1
    fi.mode = 0
    fi.talker_in = None
    with pytest.raises(qt.QtError):
        qt.qt_frame_decode(dec.model, ss, kv, fi, fo, dec.ws_ptr, dec.ws_bytes)


# ----------------------------------------------------------------- INT8 quantizer
def _gpu_quantize(torch, w_bits):
    import streaming_tts_decode_amd as qt
    rows, cols = w_bits.shape
    w = torch.from_numpy(np.ascontiguousarray(w_bits).view(np.int16)).cuda()
    q = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    qt.qt_quantize_int8(w.data_ptr(), rows, cols, q.data_ptr(), s.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def test_quantizer_edge_rows(gpu):
    import os

    import oracle
    import torch
    rows = []
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "int8_ties.txt")):
        if line.startswith("#") or not line.strip():
            continue
        rows.append(np.array([float(t) for t in line.split("|")[0].split()], dtype=np.float32))
    for r in rows:
        wb = synth._to_bf16_bits(r)[None]
        q, s = _gpu_quantize(torch, wb)
        qo, so = oracle.quantize_int8(wb)
        np.testing.assert_array_equal(q, qo)
        np.testing.assert_array_equal(s.view(np.uint32), so.view(np.uint32))
    for shape in [(3, 7), (5, 1000), (2, 257), (1, 1)]:
        wb = synth.normal_bf16(f"qedge{shape}", shape, 0.0, 0.02)
        wb[0] = 0  # an all-zero row
        q, s = _gpu_quantize(torch, wb)
        qo, so = oracle.quantize_int8(wb)
        np.testing.assert_array_equal(q, qo)
        np.testing.assert_array_equal(s.view(np.uint32), so.view(np.uint32))


def test_quantizer_bit_exact_every_decode_weight(gpu, full_weights, orc_full_i8):
    import torch
    names = synth.linear_names(synth.FULL)
    for i, name in enumerate(names):
        q, s = _gpu_quantize(torch, full_weights[name])
        qo, so = orc_full_i8.quantized[name]
        if not (np.array_equal(q, qo) and np.array_equal(s.view(np.uint32), so.view(np.uint32))):
            raise AssertionError(f"{name}: INT8 weights or scales differ from the oracle")
    log(f"[int8] {len(names)} decode weights bit-exact")


def test_int8_model_uses_quantizer_output(full_pm_i8, orc_full_i8):
    import streaming_tts_decode_amd as qt
    import torch
    for name in synth.linear_names(synth.FULL):
        qo, so = orc_full_i8.quantized[name]
        q = torch.empty(qo.shape, dtype=torch.int8, device="cuda")
        s = torch.empty(so.shape, dtype=torch.float32, device="cuda")
        qt.qt_model_export_int8(full_pm_i8.handle, name, q.data_ptr(), s.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(q.cpu().numpy(), qo, err_msg=name)
        np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32),
                                      err_msg=name)


# ----------------------------------------------------------------- fp16 range
def test_weight_beyond_half_range_is_refused(small_weights):
    """bf16 mode packs the GEMM weights as IEEE half: a weight matrix with a finite
    entry above 65504 is refused at load, naming it.  INT8 mode scales every row and
    decodes with it, but its prompt prefill runs on the unquantised weights as
    halves, so qt_prefill refuses, naming it."""
    import streaming_tts_decode_amd as qt
    from streaming_tts_decode_amd.runtime import Decoder, PackedModel
    W = dict(small_weights)
    name = "talker.layers.1.down_proj"
    w = W[name].copy()
    w[3, 17] = 0x47C3  # bf16 99840
    W[name] = w
    with pytest.raises(qt.QtError) as e:
        PackedModel(S, W, int8=False)
    assert e.value.status == 9 and name in str(e.value)
    pm8 = PackedModel(S, W, int8=True)
    try:
        dec = Decoder(pm8, batch=1, max_pages=4)
        dec.prefill_setup(16)
        dec.prefill_inputs([synth.normal_bf16("range.prompt", (5, S.talker.hidden))])
        with pytest.raises(qt.QtError) as e:
            dec.prefill()
        assert e.value.status == 9 and name in str(e.value)
    finally:
        pm8.close()


def test_activation_beyond_half_range_sets_status(small_pm):
    """A Talker input row value whose half(x * gain) overflows sets
    QT_STATUS_FP16_RANGE; the other sessions' outputs are unaffected (rows are
    independent)."""
    import streaming_tts_decode_amd as qt
    from streaming_tts_decode_amd.runtime import setup_workload
    torch = small_pm.torch
    w = small_w("Srange", batch=3, frames=1, lens=[20, 7, 41])
    x = synth.frame_inputs(w)["talker_in"][0].copy()
    dec, _ = setup_workload(w, small_pm)
    L0 = dec.kv_len.clone()
    dec.set_inputs(talker_in=x)
    dec.decode("full")
    torch.cuda.synchronize()
    assert int(dec.status.item()) == 0
    ref = dec.logits0.cpu().numpy().copy()
    x[1, 100] = 0x4843  # bf16 199680: half(199680 * gain) is inf for any gain above 0.33
    dec.kv_len.copy_(L0)
    dec.set_inputs(talker_in=x)
    dec.decode("full")
    torch.cuda.synchronize()
    st = int(dec.status.item())
    assert st & qt.STATUS_FP16_RANGE, f"status {st:#x}"
    got = dec.logits0.cpu().numpy()
    np.testing.assert_array_equal(got[[0, 2]], ref[[0, 2]])
    dec.close()
