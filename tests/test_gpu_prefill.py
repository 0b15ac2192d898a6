"""GPU checks of the prompt prefill (qt_prefill in include/qt.h) against the oracle's
prefill (oracle/__init__.py: the Talker over positions 0..T-1 from an empty
cache), through the C ABI.

For every sequence of a packed call: the codec-head logits at its last row
(parity bound: 1e-2 of the largest |logit|), the greedy codebook-0 token where the
oracle's top-2 margin is wide, the final-normed hidden state, every key and value
it stored in its pages, and decode frames that continue from the prefilled cache
(against the oracle continuing from its own prefilled cache).
"""
import numpy as np
import pytest

import synth
from tests.gpu_cases import log
from tests.parity import compare

pytestmark = pytest.mark.gpu


def _bf16(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _check_cache(dec, b, L, pre, label, dims):
    """Keys and values of session b's first L positions against the oracle's cache
    (bf16 storage: a few bf16 ulps of the per-head scale)."""
    t = dims.talker
    pages = dec.page_table_np[b, :-(-L // 16)]
    k = dec.k_pages[:, pages].cpu().numpy()  # [layers, npg, n_kv, 16, hd]
    v = dec.v_pages[:, pages].cpu().numpy()
    for name, pool, ref in (("K", k, pre["kc"]), ("V", v, pre["vc"])):
        got = _bf16(pool.view(np.uint16)).transpose(0, 1, 3, 2, 4).reshape(t.layers, -1, t.n_kv, t.head_dim)[:, :L]
        want = ref[:, :L]
        scale = np.abs(want).max(axis=(1, 3), keepdims=True)
        err = np.abs(got - want) / scale
        assert err.max() <= 2e-2, f"{label} {name}: max error {err.max():.3g} of the head scale"


def _run(pm, orc, dims, lengths, rows, max_pages, tag, frames_after=0):
    from streaming_tts_decode_amd.runtime import Decoder
    torch = pm.torch
    B = len(lengths)
    t = dims.talker
    prompts = [synth.normal_bf16(f"{tag}.prompt.s{b}", (L, t.hidden)) if L else None
               for b, L in enumerate(lengths)]
    log(f"[prefill] {tag}: lengths={lengths} rows={rows} max_pages={max_pages}")
    dec = Decoder(pm, batch=B, max_pages=max_pages)
    dec.prefill_setup(rows)
    dec.prefill_inputs(prompts)
    dec.status.zero_()
    dec.prefill()
    torch.cuda.synchronize()
    assert int(dec.status.item()) == 0
    np.testing.assert_array_equal(dec.kv_len.cpu().numpy(), lengths)
    logits = dec.pf_logits0.cpu().numpy()
    tok0 = dec.pf_tok0.cpu().numpy()
    h = _bf16(dec.pf_h.cpu().numpy().view(np.uint16))
    pres = {}
    for b, L in enumerate(lengths):
        if not L:
            assert np.all(logits[b] == 0) and np.all(h[b] == 0)
            continue
        pre = orc.prefill(prompts[b], capacity=L + frames_after)
        pres[b] = pre
        compare(logits[b][None], pre["logits0"][None], dims.cb0_range, gpu_tokens=tok0[b:b + 1],
                label=f"{tag} s{b} logits0")
        herr = np.abs(h[b] - pre["h"][-1]).max() / np.abs(pre["h"][-1]).max()
        assert herr <= 2e-2, f"{tag} s{b}: h_last error {herr:.3g}"
        _check_cache(dec, b, L, pre, f"{tag} s{b}", dims)
    if frames_after:
        x = synth.normal_bf16(f"{tag}.after", (frames_after, B, t.hidden))
        got = []
        for f in range(frames_after):
            dec.set_inputs(talker_in=x[f])
            dec.decode("talker")
            torch.cuda.synchronize()
            got.append(dec.logits0.cpu().numpy().copy())
        assert int(dec.status.item()) == 0
        for b, pre in pres.items():
            L = lengths[b]
            ref = orc.run_session("talker", frames_after, talker_in=x[:, b], length=L,
                                  cache=(pre["kc"], pre["vc"]))
            compare(np.stack([g[b] for g in got]), ref["logits0"], dims.cb0_range,
                    label=f"{tag} s{b} decode after prefill")
    return dec, prompts, logits


def test_prefill_single_sequence_and_decode_after(small_pm, orc_small):
    dec, _, _ = _run(small_pm, orc_small, synth.SMALL, [37], rows=48, max_pages=4, tag="pf1",
                     frames_after=3)
    dec.close()


def test_prefill_packed_ragged_sequences(small_pm, orc_small):
    # rows of one 16-row tile belong to two sequences (50 is not a multiple of 16),
    # an empty sequence, a sequence filling several pages, and padding rows
    dec, _, _ = _run(small_pm, orc_small, synth.SMALL, [50, 0, 77, 3], rows=192, max_pages=6,
                     tag="pf2", frames_after=2)
    dec.close()


def test_prefill_graph_replays_other_packings(small_pm):
    torch = small_pm.torch
    from streaming_tts_decode_amd.runtime import Decoder
    t = synth.SMALL.talker
    dec = Decoder(small_pm, batch=3, max_pages=8)  # 128 positions per session
    dec.prefill_setup(128)
    g = dec.prefill_capture()
    for packing in ([40, 70, 1], [0, 128, 0], [16, 16, 16]):
        prompts = [synth.normal_bf16(f"pfg.{i}.{L}", (L, t.hidden)) if L else None
                   for i, L in enumerate(packing)]
        outs = []
        for use_graph in (False, True):
            dec.prefill_inputs(prompts)
            dec.status.zero_()
            if use_graph:
                dec.replay(g)
            else:
                dec.prefill()
            torch.cuda.synchronize()  # host work between the replays
            assert int(dec.status.item()) == 0
            outs.append((dec.pf_logits0.cpu().numpy().copy(), dec.kv_len.cpu().numpy().copy(),
                         dec.k_pages.cpu().numpy().copy()))
        for a, b in zip(*outs):
            np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(outs[0][1], packing)
    dec.close()


@pytest.mark.parametrize("rows", [48, 2048])
def test_prefill_overflow_sets_status(small_pm, rows):
    # (2048 rows: the q/k pass runs in the QKV projection's epilogue)
    torch = small_pm.torch
    from streaming_tts_decode_amd import STATUS_KV_OVERFLOW
    from streaming_tts_decode_amd.runtime import Decoder
    t = synth.SMALL.talker
    dec = Decoder(small_pm, batch=1, max_pages=2)  # 32 positions
    dec.prefill_setup(rows)
    dec.prefill_inputs([synth.normal_bf16("pfo", (40, t.hidden))])
    dec.status.zero_()
    dec.prefill()
    torch.cuda.synchronize()
    assert int(dec.status.item()) & STATUS_KV_OVERFLOW
    assert np.all(np.isfinite(dec.pf_logits0.cpu().numpy()))
    dec.close()


def test_prefill_full_model(full_pm, orc_full):
    dec, _, _ = _run(full_pm, orc_full, synth.FULL, [45, 19], rows=64, max_pages=8, tag="pffull",
                     frames_after=1)
    dec.close()


def test_prefill_full_model_many_rows(full_pm, orc_full):
    # 1088 packed rows: every projection runs over 1088 activation rows at the full
    # model's matrix sizes, which selects the large-tile forms (256 x 192 for the
    # gate/up, 128 x 128 for QKV, 128 x 64 for o and down), each with a partial
    # last block of rows
    dec, _, _ = _run(full_pm, orc_full, synth.FULL, [29, 3], rows=1088, max_pages=4, tag="pfrows",
                     frames_after=1)
    dec.close()


def test_prefill_2048_rows(small_pm, orc_small):
    # 2048 rows of the small model: 128 x 128 blocks for QKV and the gate/up,
    # 128 x 64 for o and down; ragged sequences, one of a single token
    rng = np.random.default_rng(20)
    lengths = [int(x) for x in rng.integers(40, 400, size=7)] + [1]
    lengths.append(2048 - sum(lengths) - 5)
    dec, _, _ = _run(small_pm, orc_small, synth.SMALL, lengths, rows=2048, max_pages=40,
                     tag="pf2048", frames_after=1)
    dec.close()


def test_prefill_bench_prompt_first_layers(full_pm, full_weights):
    """The benchmark's prompt configuration: the full model, one 1024-token prompt in
    1024 rows (every projection in its large-tile form, the q/k pass in the QKV
    epilogue).  The keys and values of layers 0 and 1 at all 1024 positions depend
    on those layers only, so an oracle over the first two layers of the same
    weights checks them exactly as the full-depth oracle would."""
    import dataclasses
    import oracle
    from streaming_tts_decode_amd.runtime import Decoder
    d = synth.FULL
    t = d.talker
    d2 = dataclasses.replace(d, talker=dataclasses.replace(t, layers=2))
    orc2 = oracle.OracleModel(d2, full_weights)
    T = 1024
    prompt = synth.normal_bf16("pfbench.prompt", (T, t.hidden))
    log(f"[prefill] bench prompt: 1 x {T} in {T} rows, layers 0-1 against a 2-layer oracle")
    dec = Decoder(full_pm, batch=1, max_pages=T // 16)
    dec.prefill_setup(T)
    dec.prefill_inputs([prompt])
    dec.status.zero_()
    dec.prefill()
    full_pm.torch.cuda.synchronize()
    assert int(dec.status.item()) == 0
    pre = orc2.prefill(prompt, capacity=T)
    pages = dec.page_table_np[0, :T // 16]
    for name, pool, ref in (("K", dec.k_pages, pre["kc"]), ("V", dec.v_pages, pre["vc"])):
        got = _bf16(pool[:2, pages].cpu().numpy().view(np.uint16))
        got = got.transpose(0, 1, 3, 2, 4).reshape(2, T, t.n_kv, t.head_dim)
        scale = np.abs(ref).max(axis=(1, 3), keepdims=True)
        err = np.abs(got - ref[:, :T]) / scale
        log(f"[parity] bench prompt {name}: max error {err.max():.3g} of the head scale")
        assert err.max() <= 2e-2, f"bench prompt {name}: max error {err.max():.3g} of the head scale"
    dec.close()


def test_prefill_full_model_int8(full_pm_i8, orc_full_i8):
    dec, _, _ = _run(full_pm_i8, orc_full_i8, synth.FULL, [33], rows=64, max_pages=4, tag="pfi8",
                     frames_after=1)
    dec.close()


def test_prefill_largest_call(small_pm, orc_small):
    # QT_PREFILL_MAX_SEQS sequences filling QT_PREFILL_MAX_ROWS rows exactly: ragged
    # lengths, one empty sequence, one single-token sequence, and a decode frame after
    from streaming_tts_decode_amd import PREFILL_MAX_ROWS, PREFILL_MAX_SEQS
    rng = np.random.default_rng(32)
    lengths = [int(x) for x in rng.integers(16, 224, size=PREFILL_MAX_SEQS - 1)]
    lengths[5], lengths[17] = 0, 1
    lengths.append(PREFILL_MAX_ROWS - sum(lengths))
    assert 1 <= lengths[-1] < 32 * 16 and sum(lengths) == PREFILL_MAX_ROWS
    dec, _, _ = _run(small_pm, orc_small, synth.SMALL, lengths, rows=PREFILL_MAX_ROWS, max_pages=32,
                     tag="pfmax", frames_after=1)
    dec.close()
