"""Pins for the CPU oracle against closed forms, invariants, hand-worked
values and an independent brute-force recomputation (no GPU needed).

Each pin is chosen so that a plausible mistake in the oracle (a dropped
term, a wrong sign or index, a transposed operand, an off-by-one position)
fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(7)


def bf16_bits(x):
    return synth._to_bf16_bits(np.asarray(x, dtype=np.float32))


# ----------------------------------------------------------------- RMSNorm
def test_rmsnorm_constant_vector():
    n, eps = 64, 1e-6
    g = bf16_bits(rng.normal(1, 0.1, n))
    for c in (0.0, 1e-4, 0.5, -3.0, 1234.5):
        y = oracle.rmsnorm(np.full(n, c), g, eps)
        exp = c / math.sqrt(c * c + eps) * oracle.bf16_to_f64(g)
        np.testing.assert_allclose(y, exp, rtol=1e-14, atol=1e-300)


def test_rmsnorm_output_norm_and_scale():
    n, eps = 128, 1e-6
    ones = np.full(n, 0x3F80, dtype=np.uint16)
    x = rng.normal(0, 2.0, n)
    r = math.sqrt(np.mean(x * x))
    y = oracle.rmsnorm(x, ones, eps)
    assert abs(np.linalg.norm(y) - math.sqrt(n) * r / math.sqrt(r * r + eps)) < 1e-12
    # direction preserved, scale invariant up to eps
    y2 = oracle.rmsnorm(1000.0 * x, ones, eps)
    np.testing.assert_allclose(y2, y, rtol=1e-6)
    np.testing.assert_allclose(y / np.linalg.norm(y), x / np.linalg.norm(x), rtol=1e-12)


def test_rmsnorm_gain_is_elementwise():
    n = 16
    x = rng.normal(size=n)
    g = np.full(n, 0x3F80, dtype=np.uint16)
    g[3] = bf16_bits([2.0])[0]
    y1 = oracle.rmsnorm(x, np.full(n, 0x3F80, dtype=np.uint16))
    y2 = oracle.rmsnorm(x, g)
    assert y2[3] == 2.0 * y1[3]
    mask = np.arange(n) != 3
    np.testing.assert_array_equal(y2[mask], y1[mask])


# ----------------------------------------------------------------- RoPE
@pytest.mark.parametrize("d", [16, 128])
def test_rope_identity_at_zero(d):
    v = rng.normal(size=d)
    np.testing.assert_array_equal(oracle.rope(v, 0, 1e6), v)


@pytest.mark.parametrize("d", [16, 128])
def test_rope_preserves_pair_norms(d):
    v = rng.normal(size=d)
    w = oracle.rope(v, 1234, 1e6)
    h = d // 2
    np.testing.assert_allclose(np.hypot(w[:h], w[h:]), np.hypot(v[:h], v[h:]), rtol=1e-13)


@pytest.mark.parametrize("pos", [1, 7, 300, 2047])
def test_rope_first_pair_turns_by_position(pos):
    d = 128
    v = np.zeros(d)
    v[0] = 1.0
    w = oracle.rope(v, pos, 1e6)
    # rotation of (x1, x2) = (1, 0) by angle pos: (cos pos, sin pos)
    assert abs(w[0] - math.cos(pos)) < 1e-12 and abs(w[64] - math.sin(pos)) < 1e-12
    assert np.count_nonzero(np.delete(w, [0, 64])) == 0


@pytest.mark.parametrize("i", [1, 17, 63])
def test_rope_pair_frequency(i):
    d, theta, pos = 128, 1e6, 1000
    v = np.zeros(d)
    v[i] = 1.0
    w = oracle.rope(v, pos, theta)
    ang = pos * theta ** (-2.0 * i / d)
    assert abs(w[i] - math.cos(ang)) < 1e-11 and abs(w[i + 64] - math.sin(ang)) < 1e-11
    # second-half basis vector turns the same way: (0, 1) -> (-sin, cos)
    v = np.zeros(d)
    v[i + 64] = 1.0
    w = oracle.rope(v, pos, theta)
    assert abs(w[i] + math.sin(ang)) < 1e-11 and abs(w[i + 64] - math.cos(ang)) < 1e-11


def test_rope_relative_position():
    d = 128
    q, k = rng.normal(size=d), rng.normal(size=d)
    for p, pp in [(10, 3), (2000, 1999), (517, 0), (5, 9)]:
        lhs = oracle.rope(q, p, 1e6) @ oracle.rope(k, pp, 1e6)
        rhs = oracle.rope(q, p - pp, 1e6) @ k
        assert abs(lhs - rhs) < 1e-10 * (1 + abs(lhs))


# ----------------------------------------------------------------- attention
def test_attention_single_key_returns_value():
    d = 128
    q, K, V = rng.normal(size=d), rng.normal(size=(1, d)), rng.normal(size=(1, d))
    np.testing.assert_array_equal(oracle.attend(q, K, V), V[0])


def test_attention_zero_keys_average_values():
    d, n = 16, 37
    V = rng.normal(size=(n, d))
    out = oracle.attend(rng.normal(size=d), np.zeros((n, d)), V)
    np.testing.assert_allclose(out, V.mean(axis=0), rtol=1e-12, atol=1e-14)


def test_attention_two_keys_sigmoid_weights():
    d = 16
    q, K, V = rng.normal(size=d), rng.normal(size=(2, d)), rng.normal(size=(2, d))
    s = K @ q / math.sqrt(d)
    a = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    np.testing.assert_allclose(oracle.attend(q, K, V), a * V[0] + (1 - a) * V[1], rtol=1e-12)


def test_attention_scale_is_inverse_sqrt_head_dim():
    d = 64
    q = np.zeros(d)
    q[0] = 1.0
    K = np.zeros((2, d))
    K[0, 0] = math.sqrt(d) * math.log(3.0)  # score difference ln 3 -> weights 3/4, 1/4
    V = np.array([[1.0] + [0.0] * (d - 1), [0.0] * d])
    assert abs(oracle.attend(q, K, V)[0] - 0.75) < 1e-12


def test_attention_shift_invariance():
    d, n = 32, 20
    q, K, V = rng.normal(size=d), rng.normal(size=(n, d)), rng.normal(size=(n, d))
    u = rng.normal(size=d) * 5
    np.testing.assert_allclose(oracle.attend(q, K + u, V), oracle.attend(q, K, V), rtol=1e-10)


def test_gqa_equals_mha_with_repeated_heads():
    nq, nkv, d, n = 8, 4, 16, 11
    q = rng.normal(size=(nq, d))
    K, V = rng.normal(size=(n, nkv, d)), rng.normal(size=(n, nkv, d))
    g = oracle.gqa(q, K, V)
    m = oracle.gqa(q, np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1))
    np.testing.assert_array_equal(g, m)


def test_gqa_kv_head_feeds_only_its_query_pair():
    nq, nkv, d, n = 16, 8, 16, 9
    q = rng.normal(size=(nq, d))
    K, V = rng.normal(size=(n, nkv, d)), rng.normal(size=(n, nkv, d))
    base = oracle.gqa(q, K, V)
    for h in (0, 3, 7):
        K2, V2 = K.copy(), V.copy()
        K2[:, h] += 1.0
        V2[:, h] -= 2.0
        out = oracle.gqa(q, K2, V2)
        changed = np.where(np.any(out != base, axis=1))[0].tolist()
        assert changed == [2 * h, 2 * h + 1]


# ----------------------------------------------------------------- SwiGLU / argmax
def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(oracle.silu(30.0) - 30.0) < 1e-10
    assert abs(oracle.silu(-30.0)) < 1e-11
    assert oracle.silu(-30.0) < 0


def test_argmax_ties_and_nan():
    assert oracle.argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert oracle.argmax([5.0, 5.0]) == 0
    assert oracle.argmax([-1.0, -0.5, -0.5]) == 1
    assert oracle.argmax([0.0, float("nan"), 1.0]) == -1


def test_linear_matches_matrix_product():
    w = bf16_bits(rng.normal(0, 0.02, (96, 64)))
    x = rng.normal(size=64)
    np.testing.assert_allclose(oracle.linear(w, x), bf.f64(w) @ x, rtol=1e-12, atol=1e-15)
    q, s = oracle.quantize_int8(w)
    np.testing.assert_allclose(oracle.linear(w, x, q, s),
                               s.astype(np.float64) * (q.astype(np.float64) @ x), rtol=1e-12,
                               atol=1e-15)


# ----------------------------------------------------------------- INT8 quantizer
def _golden_rows():
    rows = []
    for line in open(os.path.join(GOLDEN, "int8_ties.txt")):
        if line.startswith("#") or not line.strip():
            continue
        w, s, q = line.split("|")
        rows.append((np.array([float(t) for t in w.split()], dtype=np.float32), float(s),
                     np.array([int(t) for t in q.split()], dtype=np.int8)))
    return rows


def test_int8_hand_worked_rows():
    for w, s, q in _golden_rows():
        qo, so = oracle.quantize_int8(bf16_bits(w)[None])
        assert so[0] == np.float32(s)
        np.testing.assert_array_equal(qo[0], q)


def _numpy_f32_quantize(w_bits):
    """Independent float32 path: numpy IEEE divide and numpy's half-even rint."""
    w = synth.bf16_bits_to_f32(w_bits)
    amax = np.max(np.abs(w), axis=1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s[:, None] > 0, w / s[:, None], np.float32(0))
    return np.clip(np.rint(t), -127, 127).astype(np.int8), s


@pytest.mark.parametrize("shape,std", [((64, 1024), 0.02), ((33, 2048), 1.0), ((8, 3072), 1e-3)])
def test_int8_matches_independent_float32_path(shape, std):
    w = synth.normal_bf16(f"pin.q.{shape}", shape, 0.0, std)
    q, s = oracle.quantize_int8(w)
    qn, sn = _numpy_f32_quantize(w)
    np.testing.assert_array_equal(s.view(np.uint32), sn.view(np.uint32))
    np.testing.assert_array_equal(q, qn)
    # bound |w - q s| <= s/2 (plus float32 rounding of the quotient)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    err = np.abs(wf - q.astype(np.float64) * s[:, None])
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    # the largest element of every row maps to +-127
    am = np.argmax(np.abs(wf), axis=1)
    assert np.all(np.abs(q[np.arange(len(q)), am]) == 127)


def test_int8_relative_error_order_of_magnitude():
    consts = {l.split()[0]: float(l.split()[1]) for l in open(os.path.join(GOLDEN, "page_constants.txt"))
              if not l.startswith("#")}
    w = synth.normal_bf16("pin.q.err", (256, 2048), 0.0, 0.02)
    q, s = oracle.quantize_int8(w)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    rel = np.linalg.norm(wf - q * s[:, None].astype(np.float64), axis=1) / np.linalg.norm(wf, axis=1)
    # same order of magnitude as the pages' figure (Gaussian rows: ~ 3.9 / (127 sqrt(12)))
    assert consts["int8_rel_error"] / 10 < rel.mean() < consts["int8_rel_error"] * 10


def test_page_constants_match_model_dims():
    consts = {l.split()[0]: float(l.split()[1]) for l in open(os.path.join(GOLDEN, "page_constants.txt"))
              if not l.startswith("#")}
    d = synth.FULL
    assert d.n_codebooks == consts["n_codebooks"]
    assert d.n_steps == consts["predictor_steps"]
    assert d.talker.hidden == consts["projection_in"] and d.predictor.hidden == consts["projection_out"]


# ----------------------------------------------------------------- whole frame vs brute force
def _session_inputs(d, b, L, frames):
    kb, vb = synth.gen_kv("pin", b, d.talker.layers, L, d.talker.n_kv, d.talker.head_dim)
    ti = synth.normal_bf16(f"pin.talker_in.s{b}", (frames, d.talker.hidden))
    return kb, vb, ti


@pytest.mark.parametrize("b,L", [(0, 3), (1, 9), (2, 0)])
def test_frames_match_brute_force(tiny_model, b, L):
    """B=3 ragged sessions (lengths 3, 9, 0), 3 frames each, random gains."""
    d, W, m = tiny_model
    F = 3
    kb, vb, ti = _session_inputs(d, b, L, F)
    out = m.run_session("full", F, talker_in=ti, k_bits=kb, v_bits=vb, length=L)
    lg0, hs = bf.talker_frames(W, d, bf.f64(ti), kb, vb, L)
    np.testing.assert_allclose(out["logits0"], lg0, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(out["h"], hs, rtol=1e-9, atol=1e-12)
    for f in range(F):
        tok = out["tokens"][f]
        assert tok[0] == int(np.argmax(lg0[f][: d.cb0_range]))
        lp = bf.predictor(W, d, hs[f], tok)
        np.testing.assert_allclose(out["logits_pred"][f], lp, rtol=1e-9, atol=1e-12)
        np.testing.assert_array_equal(tok[1:], np.argmax(lp, axis=1))


def test_int8_frames_match_brute_force(tiny_model):
    d, W, _ = tiny_model
    m8 = oracle.OracleModel(d, W, int8=True)
    kb, vb, ti = _session_inputs(d, 5, 6, 2)
    out = m8.run_session("full", 2, talker_in=ti, k_bits=kb, v_bits=vb, length=6)
    lg0, hs = bf.talker_frames(W, d, bf.f64(ti), kb, vb, 6, quant=m8.quantized)
    np.testing.assert_allclose(out["logits0"], lg0, rtol=1e-9, atol=1e-12)
    for f in range(2):
        lp = bf.predictor(W, d, hs[f], out["tokens"][f], quant=m8.quantized)
        np.testing.assert_allclose(out["logits_pred"][f], lp, rtol=1e-9, atol=1e-12)


def test_int8_and_bf16_frames_are_close_but_differ(tiny_model):
    d, W, m = tiny_model
    m8 = oracle.OracleModel(d, W, int8=True)
    kb, vb, ti = _session_inputs(d, 6, 4, 1)
    a = m.run_session("talker", 1, talker_in=ti, k_bits=kb, v_bits=vb, length=4)["logits0"]
    b = m8.run_session("talker", 1, talker_in=ti, k_bits=kb, v_bits=vb, length=4)["logits0"]
    rel = np.abs(a - b).max() / np.abs(a).max()
    assert 1e-5 < rel < 0.1


# ----------------------------------------------------------------- causality and composition
def test_future_cache_slots_do_not_matter(tiny_model):
    d, W, m = tiny_model
    kb, vb, ti = _session_inputs(d, 7, 5, 1)
    x = bf.f64(ti[0])[None]
    kc, vc = m.new_cache(12, kb, vb)
    y1 = m.stack_forward("talker", x, 5, kc, vc)
    kc2, vc2 = m.new_cache(12, kb, vb)
    kc2[:, 6:] = 1e3 * rng.normal(size=kc2[:, 6:].shape)
    vc2[:, 6:] = -1e3
    y2 = m.stack_forward("talker", x, 5, kc2, vc2)
    np.testing.assert_array_equal(y1, y2)


def test_predictor_step_ignores_later_tokens(tiny_model):
    d, W, m = tiny_model
    h = rng.normal(size=d.talker.hidden)
    forced = np.array([3, 1, 4, 1, 5, 9, 2, 6, 5, 3, 5, 8, 9, 7, 9, 3], dtype=np.int32)[: d.n_codebooks]
    base, _ = m.frame("predictor", h_in=h, tok0=int(forced[0]), forced=forced)
    for j in range(1, d.n_codebooks):
        f2 = forced.copy()
        f2[j] = (f2[j] + 5) % d.code_vocab
        o, _ = m.frame("predictor", h_in=h, tok0=int(forced[0]), forced=f2)
        # step s (1-based) reads forced[0 .. s-1]; steps s <= j are untouched
        np.testing.assert_array_equal(o["logits_pred"][:j], base["logits_pred"][:j])
        if j < d.n_steps:
            assert np.any(o["logits_pred"][j] != base["logits_pred"][j])


def test_zero_gate_removes_ffn(tiny_model):
    d, W, _ = tiny_model
    W1, W2 = dict(W), dict(W)
    for l in range(d.talker.layers):
        W1[f"talker.layers.{l}.gate_proj"] = np.zeros_like(W[f"talker.layers.{l}.gate_proj"])
        W2[f"talker.layers.{l}.down_proj"] = np.zeros_like(W[f"talker.layers.{l}.down_proj"])
    kb, vb, ti = _session_inputs(d, 8, 4, 1)
    o1 = oracle.OracleModel(d, W1).run_session("talker", 1, talker_in=ti, k_bits=kb, v_bits=vb, length=4)
    o2 = oracle.OracleModel(d, W2).run_session("talker", 1, talker_in=ti, k_bits=kb, v_bits=vb, length=4)
    np.testing.assert_array_equal(o1["logits0"], o2["logits0"])


def test_codebook0_argmax_skips_control_range(tiny_model):
    d, W, _ = tiny_model
    W1 = dict(W)
    head = W["talker.codec_head"].copy()
    head[d.cb0_range:] = bf16_bits(np.full(head[d.cb0_range:].shape, 0.5))  # huge control logits
    W1["talker.codec_head"] = head
    kb, vb, ti = _session_inputs(d, 9, 2, 1)
    o = oracle.OracleModel(d, W1).run_session("full", 1, talker_in=ti, k_bits=kb, v_bits=vb, length=2)
    lg = o["logits0"][0]
    assert np.argmax(lg) >= d.cb0_range
    assert o["tokens"][0][0] == int(np.argmax(lg[: d.cb0_range]))


def test_talker_and_predictor_halves_compose(tiny_model):
    d, W, m = tiny_model
    kb, vb, ti = _session_inputs(d, 10, 5, 1)
    full = m.run_session("full", 1, talker_in=ti, k_bits=kb, v_bits=vb, length=5)
    tk = m.run_session("talker", 1, talker_in=ti, k_bits=kb, v_bits=vb, length=5)
    np.testing.assert_array_equal(full["logits0"], tk["logits0"])
    pr, _ = m.frame("predictor", h_in=full["h"][0], tok0=int(full["tokens"][0][0]))
    np.testing.assert_array_equal(full["logits_pred"][0], pr["logits_pred"])
    np.testing.assert_array_equal(full["tokens"][0], pr["tokens"])


def test_teacher_forcing_with_own_tokens_is_identity(tiny_model):
    d, W, m = tiny_model
    kb, vb, ti = _session_inputs(d, 11, 3, 2)
    free = m.run_session("full", 2, talker_in=ti, k_bits=kb, v_bits=vb, length=3)
    forced = m.run_session("full", 2, talker_in=ti, k_bits=kb, v_bits=vb, length=3,
                           forced=free["tokens"])
    np.testing.assert_array_equal(free["logits_pred"], forced["logits_pred"])


def test_capacity_overflow_is_an_error(tiny_model):
    d, W, m = tiny_model
    kc, vc = m.new_cache(4)
    with pytest.raises(ValueError):
        m.stack_forward("talker", np.zeros((1, d.talker.hidden)), 4, kc, vc)


# ---------------------------------------------------------------- prefill
@pytest.mark.parametrize("T", [1, 5, 13])
def test_prefill_matches_brute_force(tiny_model, T):
    """The prompt prefill (all T positions through the stack at once, from an empty
    cache) against the brute-force full-sequence forward with an explicit causal
    mask, position by position; the codec head at the last position."""
    d, W, m = tiny_model
    X = synth.normal_bf16(f"pin.prefill.T{T}", (T, d.talker.hidden))
    out = m.prefill(X)
    h = bf.stack_forward(W, "talker", d.talker, bf.f64(X), np.arange(T))
    np.testing.assert_allclose(out["h"], h, rtol=1e-9, atol=1e-12)
    lg = bf.Lin(W, "talker.codec_head")(h[-1:])[0]
    np.testing.assert_allclose(out["logits0"], lg, rtol=1e-9, atol=1e-12)
    assert out["tok0"] == int(np.argmax(lg[: d.cb0_range]))


def test_int8_mode_prefill_keeps_bf16_weights(tiny_model):
    """INT8 quantizes the decode GEMM weights, while the prompt prefill stays BF16
    ("Qwen3-TTS Native v0.3.0", What changed): an INT8 model's prefill equals the
    bf16 model's exactly, and its decode frames do not."""
    d, W, m16 = tiny_model
    m8 = oracle.OracleModel(d, W, int8=True)
    X = synth.normal_bf16("pin.prefill.int8", (5, d.talker.hidden))
    a, b = m16.prefill(X, capacity=6), m8.prefill(X, capacity=6)
    for k in ("h", "logits0", "kc", "vc"):
        assert np.array_equal(a[k], b[k]), k
    assert a["tok0"] == b["tok0"]
    ti = synth.normal_bf16("pin.prefill.int8.next", (d.talker.hidden,))
    fa, _ = m16.frame("full", a["kc"], a["vc"], 5, talker_in=ti)
    fb, _ = m8.frame("full", b["kc"], b["vc"], 5, talker_in=ti)
    assert not np.array_equal(fa["logits0"], fb["logits0"])


def test_prefill_then_decode_equals_decoding_the_prompt(tiny_model):
    """Decode frames after a prefill of T positions see the same cache as decode
    frames after feeding the prompt one position at a time (brute force on the
    whole sequence of prompt + frame inputs)."""
    d, W, m = tiny_model
    T, F = 7, 3
    X = synth.normal_bf16("pin.prefill.cont", (T + F, d.talker.hidden))
    pre = m.prefill(X[:T], capacity=T + F)
    out = m.run_session("talker", F, talker_in=X[T:], length=T, cache=(pre["kc"], pre["vc"]))
    for f in range(F):
        h = bf.stack_forward(W, "talker", d.talker, bf.f64(X[:T + f + 1]), np.arange(T + f + 1))
        lg = bf.Lin(W, "talker.codec_head")(h[-1:])[0]
        np.testing.assert_allclose(out["logits0"][f], lg, rtol=1e-9, atol=1e-12)
