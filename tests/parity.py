"""Parity gates between the HIP path and the CPU oracle (numpy only).

Gates, per logit vector (one session, one frame, one codebook):
  * max_v |gpu_v - oracle_v| <= 1e-2 * max_v |oracle_v|  (the M* "Qwen3-TTS PR 5"
    page, Parity section, measures the logit difference relative to the logit
    scale; the tolerance is the workload's);
  * the GPU's greedy token equals the oracle's wherever the oracle's top-2 margin
    (over the argmax range) is above 1 (same page and section: agreement on
    confident positions is gated, raw argmax agreement is only reported because
    near-ties flip it).
"""
import numpy as np

REL_TOL = 1e-2
MARGIN = 1.0


def first_argmax(x):
    return np.argmax(x, axis=-1)


def compare(gpu, orc, argmax_range=None, gpu_tokens=None, label=""):
    """gpu, orc: [..., V] logits.  gpu_tokens: the GPU's own greedy tokens [...]
    (checked bit-exactly against the argmax of its own logits).  Returns a stats
    dict and asserts the gates."""
    g = np.asarray(gpu, dtype=np.float64)
    o = np.asarray(orc, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.all(np.isfinite(g)), f"{label}: non-finite GPU logits"
    r = o.shape[-1] if argmax_range is None else argmax_range
    err = np.abs(g - o).max(axis=-1)
    scale = np.abs(o).max(axis=-1)
    rel = err / scale
    srt = np.sort(o[..., :r], axis=-1)
    margin = srt[..., -1] - srt[..., -2]
    conf = margin > MARGIN
    g_tok = first_argmax(g[..., :r])
    o_tok = first_argmax(o[..., :r])
    agree = g_tok == o_tok
    if gpu_tokens is not None:
        np.testing.assert_array_equal(np.asarray(gpu_tokens), g_tok,
                                      err_msg=f"{label}: GPU tokens != argmax of GPU logits")
    tight = margin > 2 * err
    stats = {
        "label": label, "n": int(rel.size), "rel_max": float(rel.max()),
        "rel_mean": float(rel.mean()), "argmax_agree": float(agree.mean()),
        "n_confident": int(conf.sum()), "confident_agree": float(agree[conf].mean()) if conf.any() else 1.0,
        "n_margin_2err": int(tight.sum()),
    }
    print(f"[parity] {stats}", flush=True)
    assert rel.max() <= REL_TOL, f"{label}: max relative logit diff {rel.max():.4g} > {REL_TOL}"
    assert np.all(agree[conf]), f"{label}: greedy token differs at a confident position"
    assert np.all(agree[tight]), f"{label}: token differs where margin > 2 * max-abs diff"
    return stats
