"""Brute-force float64 NumPy re-computation of the decode frame, used only to
pin the CPU oracle on tiny shapes.

It is a different algorithm from the oracle's incremental decode: at every
step it recomputes the whole sequence from the first new position with
full-sequence matrix products, an explicit causal mask over
[prefilled prefix; new positions], and grouped-query attention done as
multi-head attention on key/value heads repeated along the head axis.  Nothing
is cached between steps except the given prefilled Talker keys/values.
"""
from __future__ import annotations

import numpy as np


def f64(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rms(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x, pos, theta):
    """x [..., n, d] at positions pos [n]."""
    d = x.shape[-1]
    inv = theta ** (-(2.0 * np.arange(d // 2)) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


class Lin:
    def __init__(self, W, name, quant=None):
        if quant is not None and name in quant:
            q, s = quant[name]
            self.M = q.astype(np.float64) * s.astype(np.float64)[:, None]
        else:
            self.M = f64(W[name])

    def __call__(self, x):
        return x @ self.M.T


def stack_forward(W, prefix, d, X, pos, prefix_kv=None, quant=None):
    """Full forward of n new positions X [n, H] at positions `pos` [n] (consecutive).
    prefix_kv: None or (K, V) float64 [layers, P, n_kv, hd] for positions 0..P-1.
    Returns the final-normed outputs [n, H]."""
    n = X.shape[0]
    hd, nq, nkv = d.head_dim, d.n_q, d.n_kv
    group = nq // nkv
    x = X.copy()
    P = 0 if prefix_kv is None else prefix_kv[0].shape[1]
    for l in range(d.layers):
        p = f"{prefix}.layers.{l}."
        u = rms(x, f64(W[p + "input_norm"]), d.eps)
        q = Lin(W, p + "q_proj", quant)(u).reshape(n, nq, hd).transpose(1, 0, 2)   # [nq, n, hd]
        k = Lin(W, p + "k_proj", quant)(u).reshape(n, nkv, hd).transpose(1, 0, 2)
        v = Lin(W, p + "v_proj", quant)(u).reshape(n, nkv, hd).transpose(1, 0, 2)
        q = rope(rms(q, f64(W[p + "q_norm"]), d.eps), pos, d.rope_theta)
        k = rope(rms(k, f64(W[p + "k_norm"]), d.eps), pos, d.rope_theta)
        if P:
            Kp = prefix_kv[0][l].transpose(1, 0, 2)  # [nkv, P, hd]
            Vp = prefix_kv[1][l].transpose(1, 0, 2)
            K = np.concatenate([Kp, k], axis=1)
            V = np.concatenate([Vp, v], axis=1)
        else:
            K, V = k, v
        K = np.repeat(K, group, axis=0)  # [nq, P+n, hd]
        V = np.repeat(V, group, axis=0)
        S = q @ K.transpose(0, 2, 1) / np.sqrt(hd)  # [nq, n, P+n]
        allowed = np.zeros((n, P + n), dtype=bool)
        allowed[:, :P] = True
        allowed[:, P:] = np.tril(np.ones((n, n), dtype=bool))
        S = np.where(allowed[None], S, -np.inf)
        S = S - S.max(axis=-1, keepdims=True)
        A = np.exp(S)
        A /= A.sum(axis=-1, keepdims=True)
        O = (A @ V).transpose(1, 0, 2).reshape(n, nq * hd)
        x = x + Lin(W, p + "o_proj", quant)(O)
        u = rms(x, f64(W[p + "post_norm"]), d.eps)
        g = Lin(W, p + "gate_proj", quant)(u)
        up = Lin(W, p + "up_proj", quant)(u)
        x = x + Lin(W, p + "down_proj", quant)(g / (1.0 + np.exp(-g)) * up)
    return rms(x, f64(W[prefix + ".final_norm"]), d.eps)


def predictor(W, dims, h, tokens_in, quant=None):
    """Predictor steps 1..n_steps from scratch each step.  h [Ht] float64;
    tokens_in [n_codebooks] gives the token embedded before step k as tokens_in[k-1].
    Returns logits [n_steps, code_vocab]."""
    d = dims.predictor
    p0 = Lin(W, "projection", quant)(h[None])[0]
    out = []
    for k in range(1, dims.n_codebooks):
        seq = [p0] + [f64(W[f"predictor.codec_embed.{j - 1}"])[tokens_in[j - 1]] for j in range(1, k + 1)]
        X = np.stack(seq)
        Y = stack_forward(W, "predictor", d, X, np.arange(k + 1), None, quant)
        out.append(Lin(W, f"predictor.lm_head.{k - 1}", quant)(Y[-1:])[0])
    return np.stack(out)


def talker_frames(W, dims, talker_in, k_bits, v_bits, L0, quant=None):
    """All frames of one session.  talker_in [F, Ht] float64.  Frame f recomputes
    positions L0..L0+f from scratch.  Returns (logits0 [F, V0], h [F, Ht])."""
    d = dims.talker
    kv = (f64(k_bits), f64(v_bits))
    logits, hs = [], []
    for f in range(talker_in.shape[0]):
        X = talker_in[: f + 1]
        Y = stack_forward(W, "talker", d, X, L0 + np.arange(f + 1), kv, quant)
        h = Y[-1]
        hs.append(h)
        logits.append(Lin(W, "talker.codec_head", quant)(h[None])[0])
    return np.stack(logits), np.stack(hs)
