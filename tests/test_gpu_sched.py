"""GPU checks of the lockstep scheduler (include/qt_sched.h) through the C ABI.

Invariance: decoding sessions through the scheduler -- batched into captured
sizes with padding, split into several calls per step, first frames apart, pages
appended on the fly -- gives each session what decoding it alone with plain
frames gives (the frame is an exact per-session computation; "Qwen3-TTS Native
v0.3.0", What changed: per-session state stays request-local).  The two paths
run the same kernels at different batch sizes, so they agree up to the GEMMs'
summation order; the bar is the frame's parity bound, 1e-2 of the largest
|logit| per session, frame and codebook, and tokens must agree wherever the
plain frame's top-2 margin exceeds twice the measured difference.

End of speech: the device's decision is checked against the same rule evaluated
on the host from the logits of the frames (decomputer.nl article, section 5:
the check is deferred while end of speech cannot win), with an end-of-speech
entry picked from a first run so that the decision margins are wide.
"""
import numpy as np
import pytest

import synth
from tests.gpu_cases import log

pytestmark = pytest.mark.gpu

D = synth.SMALL
PS = D.page_size


def _inputs(tag, frames, sessions, forced=True):
    t = D.talker
    x = synth.normal_bf16(f"{tag}.talker_in", (frames, sessions, t.hidden))
    rng = np.random.default_rng(synth.BASE_SEED + len(tag))
    f = np.zeros((frames, sessions, D.n_codebooks), dtype=np.int32)
    f[..., 0] = rng.integers(0, D.cb0_range, size=(frames, sessions))
    f[..., 1:] = rng.integers(0, D.code_vocab, size=(frames, sessions, D.n_codebooks - 1))
    return x, f


def _kv(tag, lengths):
    t = D.talker
    return [synth.gen_kv(tag, s, t.layers, int(L), t.n_kv, t.head_dim) for s, L in enumerate(lengths)]


def _plain(pm, kv, length, x, forced, max_pages):
    """One session decoded alone with plain frames: per-frame logits0, logits_pred, tokens."""
    from streaming_tts_decode_amd.runtime import Decoder
    torch = pm.torch
    dec = Decoder(pm, batch=1, max_pages=max_pages)
    dec.load_session_kv(0, kv[0], kv[1])
    out = {"l0": [], "lp": [], "tok": []}
    for f in range(x.shape[0]):
        dec.set_inputs(talker_in=x[f][None], forced=None if forced is None else forced[f][None])
        dec.decode("full", forced=forced is not None)
        torch.cuda.synchronize()
        out["l0"].append(dec.logits0[0].cpu().numpy().copy())
        out["lp"].append(dec.logits_pred[0].cpu().numpy().copy())
        out["tok"].append(dec.tokens[0].cpu().numpy().copy())
    assert int(dec.status.item()) == 0
    assert int(dec.kv_len[0].item()) == length + x.shape[0]
    dec.close()
    return {k: np.stack(v) for k, v in out.items()}


def _agree(got, ref, label):
    """Parity-bound comparison of one session's frames; returns the worst ratio."""
    worst = 0.0
    for f in range(ref["l0"].shape[0]):
        rows = [(ref["l0"][f], got["l0"][f], D.cb0_range)] + \
               [(ref["lp"][f][k], got["lp"][f][k], D.code_vocab) for k in range(D.n_steps)]
        for k, (r, g, rng) in enumerate(rows):
            assert np.all(np.isfinite(g)), f"{label} frame {f} codebook {k}: non-finite"
            diff = float(np.max(np.abs(g - r)))
            scale = float(np.max(np.abs(r)))
            worst = max(worst, diff / scale)
            assert diff <= 1e-2 * scale, f"{label} frame {f} codebook {k}: {diff} > 1e-2*{scale}"
            top = np.sort(r[:rng])[-2:]
            if top[1] - top[0] > 2 * diff + 1e-6:
                assert got["tok"][f][k] == ref["tok"][f][k], f"{label} frame {f} codebook {k}: token"
    return worst


def _run_sched(sch, sids, x, forced, frames):
    """Submit and step `frames` frames for every session; per-session outputs."""
    torch = sch.torch
    got = {s: {"l0": [], "lp": [], "tok": []} for s in range(len(sids))}
    groups = []
    xs = torch.from_numpy(x.view(np.int16)).to(sch.dev)
    fs = torch.from_numpy(forced).to(sch.dev) if forced is not None else None
    for f in range(frames):
        for s, sid in enumerate(sids):
            sch.submit(sid, xs[f, s], fs[f, s] if fs is not None else None)
        groups.append(sch.step())
        torch.cuda.synchronize()
        for s, sid in enumerate(sids):
            l0, lp, tok, n = sch.outputs(sid)
            assert n == f + 1
            got[s]["l0"].append(l0.cpu().numpy().copy())
            got[s]["lp"].append(lp.cpu().numpy().copy())
            got[s]["tok"].append(tok.cpu().numpy().copy())
    return {s: {k: np.stack(v) for k, v in g.items()} for s, g in got.items()}, groups


def test_sched_matches_sessions_decoded_alone(small_pm):
    from streaming_tts_decode_amd.runtime import Scheduler
    lengths = [0, 5, 16, 31, 32, 40, 47]  # empty cache, page boundaries, ragged
    frames, max_pages = 18, 5
    S = len(lengths)
    x, forced = _inputs("sched.inv", frames, S)
    kvs = _kv("sched.inv", lengths)
    log(f"[sched] invariance: S={S} lengths={lengths} frames={frames} buckets=[1,2,4]")
    sch = Scheduler(small_pm, buckets=(1, 2, 4), max_sessions=8, max_pages=max_pages,
                    num_pages=S * max_pages + 1)
    free0 = sch.free_pages()
    sids = [sch.open(L, *kvs[s]) for s, L in enumerate(lengths)]
    assert sch.free_pages() == free0 - sum(-(-L // PS) for L in lengths)
    got, groups = _run_sched(sch, sids, x, forced, frames)
    assert groups == [2] * frames  # 7 ready sessions on sizes {1,2,4}: 4 + 3 (padded to 4)
    assert sch.status() == 0
    for s, sid in enumerate(sids):
        assert sch.length(sid) == lengths[s] + frames
    # pages appended on the fly: one per page boundary crossed
    assert sch.free_pages() == free0 - sum(-(-(L + frames) // PS) for L in lengths)
    worst = 0.0
    for s, sid in enumerate(sids):
        ref = _plain(small_pm, kvs[s], lengths[s], x[:, s], forced[:, s], max_pages)
        worst = max(worst, _agree(got[s], ref, f"session {s} (L={lengths[s]})"))
    log(f"[sched] invariance: worst max|diff|/max|logit| = {worst:.2e}")
    for sid in sids:
        sch.close_session(sid)
    torch = small_pm.torch
    torch.cuda.synchronize()
    assert sch.free_pages() == free0
    sch.close()


def test_sched_group_is_bit_identical_to_plain_frame(small_pm):
    """A group of 3 sessions padded to size 4 gives, bit for bit, what a plain frame
    of the same 4-slot layout gives when its fourth slot holds an unrelated session:
    every row of the frame is computed on its own, so neither the padding nor
    anything else in the batch reaches a session."""
    from streaming_tts_decode_amd.runtime import Decoder, Scheduler
    torch = small_pm.torch
    lengths = [9, 48, 21]
    other = 37
    frames, max_pages = 5, 5
    x, forced = _inputs("sched.bit", frames, 4)
    kvs = _kv("sched.bit", lengths + [other])
    sch = Scheduler(small_pm, buckets=(4,), max_sessions=4, max_pages=max_pages)
    sids = [sch.open(L, *kvs[s]) for s, L in enumerate(lengths)]
    got, groups = _run_sched(sch, sids, x[:, :3], forced[:, :3], frames)
    assert groups == [1] * frames and sch.status() == 0
    sch.close()
    dec = Decoder(small_pm, batch=4, max_pages=max_pages)
    for b, L in enumerate(lengths + [other]):
        dec.load_session_kv(b, *kvs[b])
    for f in range(frames):
        dec.set_inputs(talker_in=x[f], forced=forced[f])
        dec.decode("full", forced=True)
        torch.cuda.synchronize()
        l0 = dec.logits0.cpu().numpy()
        lp = dec.logits_pred.cpu().numpy()
        tok = dec.tokens.cpu().numpy()
        for s in range(3):
            np.testing.assert_array_equal(got[s]["l0"][f], l0[s], err_msg=f"frame {f} session {s}")
            np.testing.assert_array_equal(got[s]["lp"][f], lp[s], err_msg=f"frame {f} session {s}")
            np.testing.assert_array_equal(got[s]["tok"][f], tok[s])
    assert int(dec.status.item()) == 0
    dec.close()
    log("[sched] bit-identical to a plain 4-slot frame")


def test_sched_first_frames_and_classes(small_pm):
    """First frames run in groups of their own ahead of running sessions; forced and
    free-running sessions never share a call; late sessions still match their
    plain decode."""
    from streaming_tts_decode_amd.runtime import Scheduler
    torch = small_pm.torch
    lengths = [20, 33, 7, 64, 1]
    frames, max_pages = 6, 6
    x, forced = _inputs("sched.cls", frames + 2, len(lengths))
    kvs = _kv("sched.cls", lengths)
    log("[sched] classes: 3 sessions, then 2 late ones; buckets=[2,4]")
    sch = Scheduler(small_pm, buckets=(2, 4), max_sessions=6, max_pages=max_pages)
    xs = torch.from_numpy(x.view(np.int16)).to(sch.dev)
    fs = torch.from_numpy(forced).to(sch.dev)
    early = [sch.open(lengths[s], *kvs[s]) for s in range(3)]
    outs = {s: {"l0": [], "lp": [], "tok": []} for s in range(5)}
    sids = list(early)
    start = {0: 0, 1: 0, 2: 0}
    for f in range(frames + 2):
        if f == 2:
            sids += [sch.open(lengths[s], *kvs[s]) for s in (3, 4)]
            start.update({3: 2, 4: 2})
        for s, sid in enumerate(sids):
            fr = f - start[s]
            # session 2 runs free, the others teacher-forced
            sch.submit(sid, xs[fr, s], None if s == 2 else fs[fr, s])
        n = sch.step()
        if f == 0:
            assert n == 2  # first frames: forced {0,1} and free {2}
        elif f == 2:
            assert n == 3  # first frames {3,4}, running forced {0,1}, running free {2}
        else:
            assert n == 2
        torch.cuda.synchronize()
        for s, sid in enumerate(sids):
            l0, lp, tok, _ = sch.outputs(sid)
            outs[s]["l0"].append(l0.cpu().numpy().copy())
            outs[s]["lp"].append(lp.cpu().numpy().copy())
            outs[s]["tok"].append(tok.cpu().numpy().copy())
    assert sch.status() == 0
    for s in range(5):
        g = {k: np.stack(v) for k, v in outs[s].items()}
        n = g["l0"].shape[0]
        tok = g["tok"]
        np.testing.assert_array_equal(tok[:, 0], np.argmax(g["l0"][:, :D.cb0_range], axis=-1))
        np.testing.assert_array_equal(tok[:, 1:], np.argmax(g["lp"], axis=-1))
        if s == 2:
            continue  # free-running: its own tokens feed back, checked for consistency only
        ref = _plain(small_pm, kvs[s], lengths[s], x[:n, s], forced[:n, s], max_pages)
        _agree(g, ref, f"session {s}")
    sch.close()


def _eos_decisions(l0, tok0, e):
    """Host evaluation of the end-of-speech rule and its margin, per frame."""
    dec, margin = [], []
    for f in range(l0.shape[0]):
        t = int(tok0[f])
        m = float(l0[f][e] - l0[f][t])
        win = e == t or (m >= 0 if e < t else m > 0)
        dec.append(win)
        margin.append(abs(m) if e != t else np.inf)
    return dec, margin


def test_sched_end_of_speech(small_pm):
    from streaming_tts_decode_amd.runtime import Scheduler
    torch = small_pm.torch
    lengths = [3, 17, 30, 45, 9, 60, 0, 24]
    frames, max_pages, min_frames = 16, 6, 4
    S = len(lengths)
    x, forced = _inputs("sched.eos", frames, S)
    kvs = _kv("sched.eos", lengths)
    log("[sched] end of speech: first run without it")
    sch = Scheduler(small_pm, buckets=(2, 8), max_sessions=S, max_pages=max_pages)
    sids = [sch.open(L, *kvs[s]) for s, L in enumerate(lengths)]
    got, _ = _run_sched(sch, sids, x, forced, frames)
    assert sch.status() == 0
    sch.close()

    # pick the entry whose decisions are widest apart and end at least one session,
    # preferring one that would also have fired before min_frames
    best = None
    for e in range(D.cb0_range, D.talker_vocab):
        ends, fires_early, ok = {}, False, True
        for s in range(S):
            dec, margin = _eos_decisions(got[s]["l0"], got[s]["tok"][:, 0], e)
            fires_early |= any(dec[:min_frames - 1])
            end = next((f + 1 for f in range(min_frames - 1, frames) if dec[f]), 0)
            upto = end if end else frames
            if min(margin[min_frames - 1:upto]) < 0.05:
                ok = False
                break
            ends[s] = end
        if ok and any(ends.values()):
            early_ends = sum(1 for v in ends.values() if 0 < v < frames)
            key = (early_ends > 0, fires_early, early_ends, sum(1 for v in ends.values() if v))
            if best is None or key > best[0]:
                best = (key, e, ends)
    assert best is not None, "no end-of-speech entry with wide decision margins"
    key, e, ends = best
    log(f"[sched] end of speech: entry {e}, expected end frames {ends}, "
        f"fires before min_frames: {key[1]}")
    assert key[0], "no entry ends a session before the last frame"

    sch = Scheduler(small_pm, buckets=(2, 8), max_sessions=S, max_pages=max_pages, eos_index=e)
    xs = torch.from_numpy(x.view(np.int16)).to(sch.dev)
    fs = torch.from_numpy(forced).to(sch.dev)
    sids = [sch.open(L, *kvs[s], min_frames=min_frames, max_frames=frames)
            for s, L in enumerate(lengths)]
    live = set(range(S))
    for f in range(frames):
        for s in sorted(live):
            sch.submit(sids[s], xs[f, s], fs[f, s])
        sch.step()
        torch.cuda.synchronize()
        for s in sorted(live):
            st, ef = sch.state(sids[s])
            if ends[s] == f + 1:
                assert (st, ef) == (2, f + 1), f"session {s}: state {st}, end {ef}"
                live.discard(s)
                with pytest.raises(Exception):
                    sch.submit(sids[s], xs[0, s], fs[0, s])
            elif f + 1 == frames:
                assert (st, ef) == (3, frames)
            else:
                assert st == 1 and ef == 0, f"session {s} frame {f + 1}: state {st}"
    assert sch.status() == 0
    sch.close()

    # pipelined: no synchronisation in the loop; a session is dropped once the host
    # has seen its end (submit refuses it), so it may decode frames past the end,
    # and the recorded end frame is still the first one that chose end of speech
    log("[sched] end of speech: pipelined pass")
    from streaming_tts_decode_amd import QtError
    sch = Scheduler(small_pm, buckets=(2, 8), max_sessions=S, max_pages=max_pages, eos_index=e)
    sids = [sch.open(L, *kvs[s], min_frames=min_frames, max_frames=frames)
            for s, L in enumerate(lengths)]
    live = set(range(S))
    for f in range(frames):
        for s in sorted(live):
            try:
                sch.submit(sids[s], xs[f, s], fs[f, s])
            except QtError as err:
                assert err.status == 7 and ends[s] and ends[s] <= f
                live.discard(s)
        sch.step()
    torch.cuda.synchronize()
    for s in range(S):
        st, ef = sch.state(sids[s])
        if ends[s]:
            assert (st, ef) == (2, ends[s]), f"session {s}: state {st}, end {ef}"
            assert sch.outputs(sids[s])[3] >= ends[s]
        else:
            assert (st, ef) == (3, frames)
    assert sch.status() == 0
    sch.close()


def test_sched_capacity_and_reuse(small_pm):
    from streaming_tts_decode_amd import QtError
    from streaming_tts_decode_amd.runtime import Scheduler
    torch = small_pm.torch
    max_pages = 2
    log("[sched] capacity: 2-page rows, pool of 4 usable pages")
    sch = Scheduler(small_pm, buckets=(1, 2), max_sessions=2, max_pages=max_pages, num_pages=5)
    kv = _kv("sched.cap", [30, 16])
    a = sch.open(30, *kv[0])
    b = sch.open(16, *kv[1])
    assert sch.free_pages() == 1
    with pytest.raises(QtError) as err:
        sch.open(0)  # both ids in use
    assert err.value.status == 6
    x, forced = _inputs("sched.cap", 4, 2)
    xs = torch.from_numpy(x.view(np.int16)).to(sch.dev)
    fs = torch.from_numpy(forced).to(sch.dev)
    # frame 1: a (30 -> 31) stays in its pages, b (16) takes the last free page
    sch.submit(a, xs[0, 0], fs[0, 0])
    sch.submit(b, xs[0, 1], fs[0, 1])
    assert sch.step() == 1
    assert sch.free_pages() == 0
    # frame 2: a (31 -> 32) still fits; frame 3 would need a third page: refused
    sch.submit(a, xs[1, 0], fs[1, 0])
    assert sch.step() == 1
    sch.submit(a, xs[2, 0], fs[2, 0])
    with pytest.raises(QtError) as err:
        sch.step()
    assert err.value.status == 6
    assert sch.length(a) == 32
    sch.close_session(a)
    torch.cuda.synchronize()
    assert sch.free_pages() == 2
    c = sch.open(20, *_kv("sched.cap2", [20])[0])
    assert c == a  # the released id is reused
    sch.submit(c, xs[3, 0], fs[3, 0])
    sch.submit(b, xs[3, 1], fs[3, 1])
    assert sch.step() == 2  # c on its first frame, b running
    torch.cuda.synchronize()
    for sid in (b, c):
        l0, lp, tok, _ = sch.outputs(sid)
        assert torch.isfinite(l0).all() and torch.isfinite(lp).all()
    assert sch.status() == 0
    sch.close()


def test_sched_sampling_is_bit_identical_to_plain_frames(small_pm):
    """Sampling sessions through the scheduler: a group of 3 padded to 4 draws, frame
    after frame, exactly what a plain 4-slot sampled frame draws with the same
    parameters, seeds and counters.  The same input every frame and a strong
    repetition penalty make the codebook-0 seen sets change the draws, so this also
    checks that each session's seen set is carried between frames.  A greedy session
    in the same steps is decoded in a call of its own."""
    from streaming_tts_decode_amd.runtime import Decoder, Scheduler
    torch = small_pm.torch
    lengths = [9, 33, 20]
    frames, max_pages = 6, 4
    params = [((0.5, 1.0, 3.0, 2), (0.8, 0.9, 1.0, 8)), ((1.0, 0.8, 2.0, 3), (1.2, 1.0, 1.0, 16)),
              ((0.7, 1.0, 4.0, 2), (0.6, 1.0, 1.0, 4))]
    seeds = [11, 12, 13]
    kvs = _kv("sched.samp", lengths + [17, 25])
    x1 = synth.normal_bf16("sched.samp.in", (1, 4, D.talker.hidden))
    xs1 = torch.from_numpy(x1.view(np.int16)).to(small_pm.dev)
    sch = Scheduler(small_pm, buckets=(4,), max_sessions=4, max_pages=max_pages, eos_index=1100)
    sids = [sch.open(L, *kvs[s], min_frames=1, max_frames=100) for s, L in enumerate(lengths)]
    for s, sid in enumerate(sids):
        sch.set_sampling(sid, params[s], seeds[s])
    greedy = sch.open(17, *kvs[3])
    got = []
    for f in range(frames):
        for s, sid in enumerate(sids):
            sch.submit(sid, xs1[0, s])
        sch.submit(greedy, xs1[0, 3])
        assert sch.step() == 2  # the sampling group and the greedy one
        torch.cuda.synchronize()
        got.append([(sch.outputs(sid)[2].cpu().numpy().copy(), sch.outputs(sid)[0].cpu().numpy().copy())
                    for sid in sids])
    for sid in sids:
        assert sch.state(sid)[0] == 1  # the end-of-speech entry never won the greedy choice here
    assert sch.status() == 0
    sch.close()
    dec = Decoder(small_pm, batch=4, max_pages=max_pages)
    for b, L in enumerate(lengths + [25]):
        dec.load_session_kv(b, *kvs[[0, 1, 2, 4][b]])
    dec.set_sampling([p[0] for p in params] + [(1.0, 1.0, 1.0, 1)],
                     [p[1] for p in params] + [(1.0, 1.0, 1.0, 1)], seeds + [0])
    changed = 0
    for f in range(frames):
        dec.set_inputs(talker_in=x1[0])
        dec.decode("full", sampling=True)
        torch.cuda.synchronize()
        tok = dec.tokens.cpu().numpy()
        l0 = dec.logits0.cpu().numpy()
        for s in range(3):
            np.testing.assert_array_equal(got[f][s][0], tok[s], err_msg=f"frame {f} session {s}")
            np.testing.assert_array_equal(got[f][s][1], l0[s], err_msg=f"frame {f} session {s}")
        changed += int(np.any(tok[:3, 0] != np.stack([got[0][s][0][0] for s in range(3)])))
    assert int(dec.status.item()) == 0
    dec.close()
    log(f"[sched] sampled scheduler frames bit-identical to plain frames; "
        f"frames whose codebook-0 draws moved off the first frame's: {changed}")


def test_prefill_into_scheduler_pages_then_steps(small_pm, orc_small):
    """Prompts prefilled (qt_prefill) straight into the pages the scheduler hands out,
    then teacher-forced frames through qt_sched_step: every session's codec-head
    logits after the prefill and every frame's logits match the oracle continuing
    from its own prefill ("Qwen3-TTS PR 5", What changed: the Talker prefill, then
    decode from its cache)."""
    from streaming_tts_decode_amd.runtime import Scheduler
    from tests.parity import compare
    torch = small_pm.torch
    lengths = [37, 16, 1, 60, 33]  # a page boundary, one token, several pages
    F = 3
    S = len(lengths)
    x, forced = _inputs("sched.pf", F, S)
    prompts = [synth.normal_bf16(f"sched.pf.prompt{s}", (L, D.talker.hidden)) for s, L in enumerate(lengths)]
    sch = Scheduler(small_pm, buckets=(1, 2, 4), max_sessions=8, max_pages=8)
    try:
        sess = [sch.open_pages(L) for L in lengths]
        assert [len(p) for _, p in sess] == [-(-L // PS) for L in lengths]
        l0, tok0, _, st = sch.prefill(sess, prompts)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        got, groups = _run_sched(sch, [sid for sid, _ in sess], x, forced, F)
        assert sch.status() == 0
        for s, sid in enumerate(sess):
            assert sch.length(sid[0]) == lengths[s] + F
        log(f"[sched] prefill then steps: lengths {lengths}, groups per step {groups}")
        worst = 0.0
        for s, L in enumerate(lengths):
            pre = orc_small.prefill(prompts[s], capacity=L + F)
            st0 = compare(l0[s].cpu().numpy()[None], pre["logits0"][None], D.cb0_range,
                          gpu_tokens=tok0[s:s + 1].cpu().numpy(), label=f"sched prefill s{s}")
            ref = orc_small.run_session("full", F, talker_in=x[:, s], length=L,
                                        forced=forced[:, s], cache=(pre["kc"], pre["vc"]))
            a = compare(got[s]["l0"], ref["logits0"], D.cb0_range, gpu_tokens=got[s]["tok"][:, 0],
                        label=f"sched after prefill s{s} logits0")
            b = compare(got[s]["lp"], ref["logits_pred"], D.code_vocab, gpu_tokens=got[s]["tok"][:, 1:],
                        label=f"sched after prefill s{s} predictor")
            worst = max(worst, st0["rel_max"], a["rel_max"], b["rel_max"])
        log(f"[sched] prefill then steps: worst relative logit error {worst:.3g}")
    finally:
        sch.close()


def test_sched_inputs_from_another_stream(small_pm):
    """Inputs allocated on another stream and dropped by the caller right after
    submit are still intact when the scheduler's stream reads them: the step is
    held back behind a busy kernel while the other stream allocates and fills new
    tensors of the same size, which the caching allocator would otherwise place in
    the dropped inputs' memory."""
    from streaming_tts_decode_amd.runtime import Scheduler
    torch = small_pm.torch
    lengths = [13, 40]
    frames, max_pages = 3, 5
    x, forced = _inputs("sched.stream", frames, len(lengths))
    kvs = _kv("sched.stream", lengths)
    sch = Scheduler(small_pm, buckets=(2,), max_sessions=2, max_pages=max_pages)
    sids = [sch.open(L, *kvs[s]) for s, L in enumerate(lengths)]
    side = torch.cuda.Stream()
    got = {s: {"l0": [], "lp": [], "tok": []} for s in range(len(sids))}
    for f in range(frames):
        with torch.cuda.stream(sch.stream):
            torch.cuda._sleep(20_000_000)  # holds the step back (bounded busy loop)
        with torch.cuda.stream(side):
            xs = torch.from_numpy(x[f].view(np.int16)).to(sch.dev)
            fs = torch.from_numpy(forced[f]).to(sch.dev)
        side.synchronize()
        for s, sid in enumerate(sids):
            sch.submit(sid, xs[s], fs[s])
        del xs, fs
        sch.step()
        with torch.cuda.stream(side):  # same sizes, garbage contents
            junk_x = torch.full((len(lengths), D.talker.hidden), 0x7bff, dtype=torch.int16, device=sch.dev)
            junk_f = torch.full((len(lengths), D.n_codebooks), 7, dtype=torch.int32, device=sch.dev)
        torch.cuda.synchronize()
        del junk_x, junk_f
        for s, sid in enumerate(sids):
            l0, lp, tok, n = sch.outputs(sid)
            assert n == f + 1
            got[s]["l0"].append(l0.cpu().numpy().copy())
            got[s]["lp"].append(lp.cpu().numpy().copy())
            got[s]["tok"].append(tok.cpu().numpy().copy())
    assert sch.status() == 0
    sch.close()
    for s in range(len(lengths)):
        ref = _plain(small_pm, kvs[s], lengths[s], x[:, s], forced[:, s], max_pages)
        _agree({k: np.stack(v) for k, v in got[s].items()}, ref, f"session {s}")
    log("[sched] inputs from another stream intact")
