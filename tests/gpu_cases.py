"""Shared GPU-vs-oracle case runner (used by the gpu-marked tests).

The GPU always decodes the whole batch in the workload's launch configuration
(eager frames, or one captured graph replayed once per frame).  The oracle,
which is slow, recomputes a chosen subset of sessions over every frame; the
GPU's other sessions get seeded random forced tokens and are checked through
properties only (finite logits, tokens equal to the argmax of their logits,
kv_len advanced).  Sessions are independent, so a checked session sees exactly
the inputs the oracle saw.
"""
import sys

import numpy as np

import synth
from tests.parity import compare


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_frames(pm, orc, w, check, use_graph=None, kv_seed_tag=None):
    """Run workload w on PackedModel pm; compare sessions `check` with oracle orc.
    Returns a list of stats dicts."""
    from streaming_tts_decode_amd.runtime import setup_workload
    torch = pm.torch
    d = w.dims
    t = d.talker
    tag = kv_seed_tag or w.name
    use_graph = w.graph if use_graph is None else use_graph
    inputs = synth.frame_inputs(w)
    lengths = w.lengths()
    check = sorted(set(int(b) for b in check))
    log(f"[case] {w.name}: mode={w.mode} B={w.batch} frames={w.frames} int8={pm.int8} "
        f"graph={use_graph} check={check} L={lengths.tolist()[:8]}...")

    kv_pool = {}
    if w.mode != "predictor":
        for b in check:
            kv_pool[b] = synth.gen_kv(tag, b, t.layers, int(lengths[b]), t.n_kv, t.head_dim)
    orc_out = {}
    for b in check:
        if w.mode == "predictor":
            orc_out[b] = orc.run_session("predictor", w.frames, h_in=inputs["h_in"][:, b],
                                         tok0=inputs["tok0"][:, b])
        else:
            kb, vb = kv_pool[b]
            orc_out[b] = orc.run_session(w.mode, w.frames, talker_in=inputs["talker_in"][:, b],
                                         k_bits=kb, v_bits=vb, length=int(lengths[b]))
    log(f"[case] {w.name}: oracle done")

    dec, _ = setup_workload(w, pm, kv_pool=kv_pool)
    rng = np.random.default_rng(99)
    forced = rng.integers(0, d.cb0_range, size=(w.frames, w.batch, d.n_codebooks)).astype(np.int32)
    forced[..., 1:] = rng.integers(0, d.code_vocab, size=(w.frames, w.batch, d.n_codebooks - 1))
    for b in check:
        forced[:, b] = orc_out[b]["tokens"]
    if w.mode == "predictor":
        forced[:, :, 0] = inputs["tok0"]
    dec.status.zero_()
    graph = dec.capture(w.mode, forced=True) if use_graph else None
    got = {k: [] for k in ("logits0", "logits_pred", "tokens")}
    for f in range(w.frames):
        if w.mode == "predictor":
            dec.set_inputs(h_in=inputs["h_in"][f], tok0=inputs["tok0"][f], forced=forced[f])
        else:
            dec.set_inputs(talker_in=inputs["talker_in"][f], forced=forced[f])
        if graph is not None:
            dec.replay(graph)
        else:
            dec.decode(w.mode, forced=True)
        torch.cuda.synchronize()
        got["logits0"].append(dec.logits0.cpu().numpy().copy())
        got["logits_pred"].append(dec.logits_pred.cpu().numpy().copy())
        got["tokens"].append(dec.tokens.cpu().numpy().copy())
    got = {k: np.stack(v) for k, v in got.items()}  # [frames, B, ...]
    status = int(dec.status.cpu().item())
    kv_end = dec.kv_len.cpu().numpy()
    dec.close()
    log(f"[case] {w.name}: gpu done, status={status}")
    assert status == 0, f"device status bits {status:#x}"
    if w.mode != "predictor":
        np.testing.assert_array_equal(kv_end, lengths + w.frames)

    # every session: finite logits, tokens = argmax of own logits
    stats = []
    if w.mode != "predictor":
        lg0 = got["logits0"]
        assert np.all(np.isfinite(lg0))
        np.testing.assert_array_equal(got["tokens"][..., 0], np.argmax(lg0[..., :d.cb0_range], axis=-1))
    if w.mode != "talker":
        lp = got["logits_pred"]
        assert np.all(np.isfinite(lp))
        np.testing.assert_array_equal(got["tokens"][..., 1:], np.argmax(lp, axis=-1))
    for b in check:
        o = orc_out[b]
        if w.mode != "predictor":
            stats.append(compare(got["logits0"][:, b], o["logits0"], d.cb0_range,
                                 label=f"{w.name} s{b} talker"))
        if w.mode != "talker":
            stats.append(compare(got["logits_pred"][:, b], o["logits_pred"],
                                 label=f"{w.name} s{b} predictor"))
    return stats
