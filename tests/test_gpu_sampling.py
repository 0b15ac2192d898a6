"""GPU checks of the frame's token draws (qt_sampling in include/qt.h) against the
sampling oracle (oracle/sampler.py), through the C ABI.

Every draw is compared on identical inputs: the oracle sampler runs on the
logits the GPU frame itself produced (copied back), with the same parameters,
seen set and Philox draw u.  The oracle's scores and sums are float64 and the
kernel's float32, so the two may differ only where the decision sits within
float32 rounding of one of its boundaries (u against a running sum, the top-p
cut, the top-k cut); the test demands exact agreement everywhere else and a
valid candidate there, and counts such ties.
"""
import numpy as np
import pytest

import synth
from oracle import sampler
from tests.gpu_cases import log

pytestmark = pytest.mark.gpu

D = synth.SMALL
GAP = 1e-5  # relative closeness to a boundary below which float32 and float64 may differ


def _decoder(pm, lengths, max_pages=6, tag="samp"):
    from streaming_tts_decode_amd.runtime import Decoder
    t = D.talker
    dec = Decoder(pm, batch=len(lengths), max_pages=max_pages)
    for b, L in enumerate(lengths):
        dec.load_session_kv(b, *synth.gen_kv(tag, b, t.layers, int(L), t.n_kv, t.head_dim))
    return dec


def _params(B, rng):
    """Per-session (temperature, top_p, penalty, top_k): a spread including the
    edges (top_k 1 and 64, top_p 1, penalty 1)."""
    talker, pred = [], []
    for b in range(B):
        talker.append((float(rng.choice([0.6, 0.9, 1.0, 1.3])), float(rng.choice([1.0, 0.9, 0.7])),
                       float(rng.choice([1.0, 1.05, 1.5])), int(rng.choice([1, 5, 50, 64]))))
        pred.append((float(rng.choice([0.7, 0.9, 1.2])), float(rng.choice([1.0, 0.8])), 1.0,
                     int(rng.choice([2, 17, 50, 64]))))
    return talker, pred


def _check_draw(logits, tok, u, prm, seen, label, stats):
    T, p, r, k = prm
    want, det = sampler.sample(logits, u, temperature=T, top_k=k, top_p=p, penalty=r, seen=seen)
    # scores are O(1..10): float32 rounds them by ~1e-6, far below 1e-4
    tied = det["u_gap"] < GAP or det["p_gap"] < GAP or det["k_gap"] < 1e-4
    stats["n"] += 1
    if tok == want:
        stats["exact"] += 1
        return
    assert tied, f"{label}: GPU drew {tok}, oracle {want} (u={u}, gaps {det['u_gap']:.2e} " \
                 f"{det['p_gap']:.2e} {det['k_gap']:.2e})"
    assert tok in det["cand"][:det["kept"] + 1], f"{label}: GPU token {tok} is no candidate"
    stats["tied"] += 1


def _frames(dec, frames, x, forced=None, mode="full", h=None, tok0=None):
    """Run frames with sampling; per frame: (counter, seen before, logits0, logits_pred, tokens)."""
    torch = dec.torch
    out = []
    for f in range(frames):
        if mode == "predictor":
            dec.set_inputs(h_in=h[f], tok0=tok0[f], forced=None if forced is None else forced[f])
        else:
            dec.set_inputs(talker_in=x[f], forced=None if forced is None else forced[f])
        ctr = dec.kv_len.cpu().numpy().copy()
        seen = dec.seen0.cpu().numpy().copy()
        dec.decode(mode, forced=forced is not None, sampling=True)
        torch.cuda.synchronize()
        out.append((ctr, seen, dec.logits0.cpu().numpy().copy(), dec.logits_pred.cpu().numpy().copy(),
                    dec.tokens.cpu().numpy().copy()))
    return out


def _seen_bits(words, n):
    bits = np.unpackbits(words.view(np.uint8), bitorder="little")
    return bits[:n].astype(bool)


def _verify(out, talker, pred, seeds, label, stats, mode="full"):
    for f, (ctr, seen, l0, lp, tok) in enumerate(out):
        for b in range(tok.shape[0]):
            if mode != "predictor":
                u = sampler.uniform(seeds[b], int(ctr[b]), 0)
                _check_draw(l0[b, :D.cb0_range], int(tok[b, 0]), u, talker[b],
                            _seen_bits(seen[b], D.cb0_range), f"{label} f{f} s{b} cb0", stats)
            if mode == "talker":
                assert np.all(tok[b, 1:] == -1)
                continue
            for k in range(1, D.n_codebooks):
                u = sampler.uniform(seeds[b], int(ctr[b]), k)
                _check_draw(lp[b, k - 1], int(tok[b, k]), u, pred[b], None,
                            f"{label} f{f} s{b} cb{k}", stats)


def test_draws_match_oracle_sampler(small_pm):
    rng = np.random.default_rng(7)
    lengths = [5, 16, 33, 47, 2, 60]
    B, frames = len(lengths), 6
    dec = _decoder(small_pm, lengths)
    talker, pred = _params(B, rng)
    seeds = [int(s) for s in rng.integers(0, 2 ** 63, size=B)]
    dec.set_sampling(talker, pred, seeds)
    # sessions start with some codebook-0 tokens already seen
    seen0 = np.zeros((B, (D.cb0_range + 31) // 32), dtype=np.uint32)
    seen0[:, :4] = rng.integers(0, 2 ** 32, size=(B, 4), dtype=np.uint64).astype(np.uint32)
    dec.seen0.copy_(dec.torch.from_numpy(seen0.view(np.int32)))
    x = synth.normal_bf16("samp.in", (frames, B, D.talker.hidden))
    forced = rng.integers(0, D.code_vocab, size=(frames, B, D.n_codebooks)).astype(np.int32)
    forced[..., 0] = rng.integers(0, D.cb0_range, size=(frames, B))
    log(f"[sampling] B={B} frames={frames} talker params {talker} predictor {pred}")
    stats = {"n": 0, "exact": 0, "tied": 0}
    out = _frames(dec, frames, x, forced=forced)
    _verify(out, talker, pred, seeds, "forced", stats)
    # the seen sets gained exactly the drawn codebook-0 tokens
    final_seen = dec.seen0.cpu().numpy().view(np.uint32)
    want = seen0.copy()
    for f in range(frames):
        for b in range(B):
            t0 = int(out[f][4][b, 0])
            want[b, t0 >> 5] |= np.uint32(1 << (t0 & 31))
    np.testing.assert_array_equal(final_seen, want)
    assert int(dec.status.item()) == 0
    np.testing.assert_array_equal(dec.kv_len.cpu().numpy(), np.array(lengths) + frames)
    log(f"[sampling] {stats}")
    assert stats["exact"] >= 0.99 * stats["n"]
    dec.close()


def test_drawn_tokens_feed_the_next_step(small_pm):
    """Free-running: the predictor embeds its own draws.  Re-running the same frames
    teacher-forced with those draws must give bit-identical logits and draws."""
    torch = small_pm.torch
    rng = np.random.default_rng(11)
    lengths = [9, 30, 21]
    B, frames = len(lengths), 4
    x = synth.normal_bf16("samp.feed", (frames, B, D.talker.hidden))
    talker, pred = _params(B, rng)
    seeds = [1, 2, 3]
    runs = []
    for forced in (None, "own"):
        dec = _decoder(small_pm, lengths, tag="feed")
        dec.set_sampling(talker, pred, seeds)
        f_arr = None if forced is None else np.stack([o[4] for o in runs[0]])
        runs.append(_frames(dec, frames, x, forced=f_arr))
        assert int(dec.status.item()) == 0
        dec.close()
    for f in range(frames):
        for i in (2, 3, 4):
            np.testing.assert_array_equal(runs[0][f][i], runs[1][f][i])
    stats = {"n": 0, "exact": 0, "tied": 0}
    _verify(runs[0], talker, pred, seeds, "free", stats)
    log(f"[sampling] free-running {stats}")


def test_top_k_one_equals_greedy_and_seeds_repeat(small_pm):
    torch = small_pm.torch
    lengths = [12, 40, 3, 25]
    B = len(lengths)
    x = synth.normal_bf16("samp.greedy", (1, B, D.talker.hidden))
    dec = _decoder(small_pm, lengths, tag="greedy")
    L0 = dec.kv_len.clone()
    dec.set_inputs(talker_in=x[0])
    dec.decode("full")
    torch.cuda.synchronize()
    greedy = dec.tokens.cpu().numpy().copy()
    dec.kv_len.copy_(L0)
    dec.set_sampling((0.8, 0.9, 1.3, 1), (1.1, 0.5, 1.0, 1), [5, 6, 7, 8])
    dec.decode("full", sampling=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dec.tokens.cpu().numpy(), greedy)
    # the same seeds and counters repeat exactly; other seeds draw differently
    dec.set_sampling((1.0, 1.0, 1.0, 64), (1.0, 1.0, 1.0, 64), [5, 6, 7, 8])
    draws = []
    for seeds in ([5, 6, 7, 8], [5, 6, 7, 8], [9, 10, 11, 12]):
        dec.kv_len.copy_(L0)
        dec.seen0.zero_()
        dec.set_sampling((1.0, 1.0, 1.0, 64), (1.0, 1.0, 1.0, 64), seeds)
        dec.decode("full", sampling=True)
        torch.cuda.synchronize()
        draws.append(dec.tokens.cpu().numpy().copy())
    np.testing.assert_array_equal(draws[0], draws[1])
    assert np.mean(draws[0] != draws[2]) > 0.5
    assert int(dec.status.item()) == 0
    dec.close()


def test_talker_and_predictor_modes(small_pm):
    rng = np.random.default_rng(5)
    lengths = [7, 19]
    B, frames = 2, 3
    talker, pred = _params(B, rng)
    seeds = [77, 78]
    dec = _decoder(small_pm, lengths, tag="modes")
    dec.set_sampling(talker, pred, seeds)
    x = synth.normal_bf16("samp.modes", (frames, B, D.talker.hidden))
    stats = {"n": 0, "exact": 0, "tied": 0}
    out = _frames(dec, frames, x, mode="talker")
    _verify(out, talker, pred, seeds, "talker", stats, mode="talker")
    np.testing.assert_array_equal(dec.kv_len.cpu().numpy(), np.array(lengths) + frames)
    h = synth.normal_bf16("samp.h", (frames, B, D.talker.hidden))
    tok0 = rng.integers(0, D.cb0_range, size=(frames, B)).astype(np.int32)
    out = _frames(dec, frames, None, mode="predictor", h=h, tok0=tok0)
    for f in range(frames):
        np.testing.assert_array_equal(out[f][4][:, 0], tok0[f])
    _verify(out, talker, pred, seeds, "predictor", stats, mode="predictor")
    assert int(dec.status.item()) == 0
    log(f"[sampling] modes {stats}")
    dec.close()


def test_bad_parameters_fall_back_to_greedy(small_pm):
    torch = small_pm.torch
    from streaming_tts_decode_amd import STATUS_BAD_SAMPLER
    lengths = [10, 20]
    x = synth.normal_bf16("samp.bad", (1, 2, D.talker.hidden))
    dec = _decoder(small_pm, lengths, tag="bad")
    L0 = dec.kv_len.clone()
    dec.set_inputs(talker_in=x[0])
    dec.decode("full")
    torch.cuda.synchronize()
    greedy = dec.tokens.cpu().numpy().copy()
    dec.kv_len.copy_(L0)
    # session 0: top_k 65 and temperature 0; session 1: top_p 0 and penalty 0.5
    dec.set_sampling([(0.0, 1.0, 1.0, 65), (1.0, 0.0, 0.5, 5)],
                     [(1.0, 1.0, 1.0, 0), (-1.0, 1.0, 1.0, 3)], [1, 2])
    dec.decode("full", sampling=True)
    torch.cuda.synchronize()
    assert int(dec.status.item()) == STATUS_BAD_SAMPLER
    np.testing.assert_array_equal(dec.tokens.cpu().numpy(), greedy)
    dec.close()


def test_sampled_graph_replays_match_eager(small_pm):
    torch = small_pm.torch
    rng = np.random.default_rng(9)
    lengths = [14, 29, 40]
    B, frames = 3, 4
    talker, pred = _params(B, rng)
    x = synth.normal_bf16("samp.graph", (frames, B, D.talker.hidden))
    res = []
    for use_graph in (False, True):
        dec = _decoder(small_pm, lengths, tag="graph")
        dec.set_sampling(talker, pred, [3, 4, 5])
        g = dec.capture("full", sampling=True) if use_graph else None
        toks = []
        for f in range(frames):
            dec.set_inputs(talker_in=x[f])
            if g:
                dec.replay(g)
            else:
                dec.decode("full", sampling=True)
            torch.cuda.synchronize()  # eager host work between replays
            toks.append((dec.tokens.cpu().numpy().copy(), dec.logits_pred.cpu().numpy().copy()))
        res.append(toks)
        assert int(dec.status.item()) == 0
        dec.close()
    for f in range(frames):
        np.testing.assert_array_equal(res[0][f][0], res[1][f][0])
        np.testing.assert_array_equal(res[0][f][1], res[1][f][1])


def _sample_rows(torch, logits, params, seeds, counters, codebook=0, seen=None):
    """qt_sample on host arrays; returns (tokens, seen after, status)."""
    import streaming_tts_decode_amd as qt
    R, V = logits.shape
    dev = torch.device("cuda")
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(dev)
    rec = np.zeros(R, dtype=[("t", "<f4"), ("p", "<f4"), ("r", "<f4"), ("k", "<i4")])
    for i, (t, p, r, k) in enumerate(params):
        rec[i] = (t, p, r, k)
    pr = torch.from_numpy(rec.view(np.int32).reshape(R, 4).copy()).to(dev)
    sd = torch.from_numpy(np.asarray(seeds, dtype=np.uint64).view(np.int64)).to(dev)
    ct = torch.from_numpy(np.asarray(counters, dtype=np.int32)).to(dev)
    words = (V + 31) // 32
    sn = None
    if seen is not None:
        packed = np.zeros((R, words * 32), dtype=bool)
        packed[:, :V] = seen
        sn = torch.from_numpy(np.packbits(packed, axis=1, bitorder="little").view(np.int32).copy()).to(dev)
    tok = torch.zeros(R, dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    qt.qt_sample(lg.data_ptr(), R, V, V, pr.data_ptr(), sd.data_ptr(), ct.data_ptr(), codebook,
                 sn.data_ptr() if sn is not None else None, tok.data_ptr(), st.data_ptr(),
                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    after = None
    if sn is not None:
        after = np.unpackbits(sn.cpu().numpy().view(np.uint8), axis=1, bitorder="little")[:, :V].astype(bool)
    return tok.cpu().numpy(), after, int(st.item())


def _check_rows(logits, toks, params, seeds, counters, codebook, seen, label):
    stats = {"n": 0, "exact": 0, "tied": 0}
    for r in range(logits.shape[0]):
        u = sampler.uniform(seeds[r], int(counters[r]), codebook)
        _check_draw(logits[r], int(toks[r]), u, params[r], None if seen is None else seen[r],
                    f"{label} row {r}", stats)
    return stats


def test_sampler_rows_edge_cases(gpu):
    """Rows that stress the top-k selection: random rows, all-equal rows (every entry
    ties with the k-th), rows of three distinct values (massive ties at the k-th
    value, ranked by index), NaN and -inf entries, rows shorter than top_k, a
    huge-scale row, the longest row (4096)."""
    import torch
    rng = np.random.default_rng(21)
    cases = []
    V = 2048
    cases.append(("normal", rng.normal(scale=1.5, size=(24, V)).astype(np.float32)))
    cases.append(("equal", np.full((6, V), 0.37, dtype=np.float32)))
    cases.append(("three values", rng.integers(0, 3, size=(8, V)).astype(np.float32)))
    x = rng.normal(size=(6, V)).astype(np.float32)
    x[:, ::7] = np.nan
    x[:, 3::11] = -np.inf
    cases.append(("nan and -inf", x))
    cases.append(("huge scale", (rng.normal(size=(4, V)) * 1e4).astype(np.float32)))
    cases.append(("short rows", rng.normal(size=(6, 40)).astype(np.float32)))
    cases.append(("longest rows", rng.normal(size=(4, 4096)).astype(np.float32)))
    total = {"n": 0, "exact": 0, "tied": 0}
    for label, lg in cases:
        R = lg.shape[0]
        params = [(float(rng.choice([0.5, 1.0, 1.7])), float(rng.choice([1.0, 0.9, 0.5])), 1.0,
                   int(rng.choice([1, 7, 50, 64]))) for _ in range(R)]
        seeds = [int(s) for s in rng.integers(0, 2 ** 62, size=R)]
        counters = rng.integers(0, 10000, size=R).astype(np.int32)
        toks, _, status = _sample_rows(torch, lg, params, seeds, counters, codebook=3)
        assert status == 0, label
        st = _check_rows(lg, toks, params, seeds, counters, 3, None, label)
        for k in total:
            total[k] += st[k]
    log(f"[sampling] edge-case rows {total}")
    assert total["exact"] >= total["n"] - 2


def test_sampler_rows_many_draws_and_penalty(gpu):
    """One row drawn under 2000 counters matches the oracle draw by draw (so its
    frequencies are the oracle's distribution); a repetition penalty over a seen set
    changes the draws as the oracle's does, and each row's draw joins its set."""
    import torch
    rng = np.random.default_rng(5)
    V = 256
    row = rng.normal(scale=2.0, size=V).astype(np.float32)
    n = 2000
    lg = np.tile(row, (n, 1))
    params = [(0.8, 0.9, 1.0, 20)] * n
    seeds = [77] * n
    counters = np.arange(n, dtype=np.int32)
    toks, _, status = _sample_rows(torch, lg, params, seeds, counters)
    assert status == 0
    st = _check_rows(lg, toks, params, seeds, counters, 0, None, "draws")
    assert st["exact"] >= n - 2
    p = sampler.distribution(row, temperature=0.8, top_k=20, top_p=0.9)
    freq = np.bincount(toks, minlength=V) / n
    assert np.abs(freq - p).max() < 0.05
    # penalty over a seen set that holds the most probable entries
    seen = np.zeros((n, V), dtype=bool)
    seen[:, np.argsort(-row)[:5]] = True
    params = [(0.8, 1.0, 3.0, 20)] * n
    toks2, after, status = _sample_rows(torch, lg, params, seeds, counters, seen=seen)
    assert status == 0
    st = _check_rows(lg, toks2, params, seeds, counters, 0, seen, "penalty")
    assert st["exact"] >= n - 2
    assert np.mean(toks2 != toks) > 0.2
    want = seen.copy()
    want[np.arange(n), toks2] = True
    np.testing.assert_array_equal(after, want)


def test_sampler_rows_bad_parameters(gpu):
    import torch
    from streaming_tts_decode_amd import STATUS_BAD_SAMPLER
    rng = np.random.default_rng(8)
    lg = rng.normal(size=(3, 512)).astype(np.float32)
    lg[2, 100] = lg[2, 200] = lg[2].max() + 1.0  # tie: the lower index wins
    params = [(0.0, 1.0, 1.0, 5), (1.0, 1.0, 1.0, 65), (1.0, 0.0, 1.0, 5)]
    toks, _, status = _sample_rows(torch, lg, params, [1, 2, 3], [0, 0, 0])
    assert status == STATUS_BAD_SAMPLER
    np.testing.assert_array_equal(toks, np.argmax(lg, axis=1))
    assert toks[2] == 100
