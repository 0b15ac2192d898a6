"""Sampling oracle: the codec-token sampler of one decode frame, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the plain reference the
HIP path's sampler is checked against.  Only ``tests/``, ``__graft_entry__`` and
``bench.py``'s CPU baseline may import it.

What the pages fix ("Qwen3-TTS PR 5", Graph: two samplers, the codebook-0 one with
a repetition penalty; "Qwen3-TTS Native v0.3.0", What changed: sampling state,
seen-token histories and random states are per request; the smoke results: seeded
runs repeat byte for byte) and the readings taken where they are silent:

 1. Codebook 0 draws over entries [0, cb0_range) of the codec head; predictor
    step k draws over its head's code_vocab entries.
 2. Repetition penalty (codebook 0 only) over the session's set of codebook-0
    tokens emitted so far: a seen entry's logit x becomes x / theta if x > 0,
    else x * theta (the CTRL paper's form, Keskar et al. 2019).
 3. Temperature: z = x / T.
 4. Top-k: the k largest z, ties to the lower index.
 5. Top-p: candidates in order (z descending, index ascending) with weights
    w_j = exp(z_j - z_max); the shortest prefix whose weight sum reaches
    top_p times the candidates' total is kept (at least one).
 6. Draw: r = u * (kept total); the token is the first kept candidate whose
    running sum exceeds r.
 7. u comes from Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC 2011) with key (seed, 0) and counter
    (frame counter, codebook, 0, 0): the top 24 bits of the first output word,
    times 2^-24, so u is exact in float32 and lies in [0, 1).
"""
from __future__ import annotations

import math

import numpy as np

_M64 = (1 << 64) - 1
# Philox4x64 round multipliers and Weyl key increments (Salmon et al. 2011, Table 2
# and section 4.2): the golden ratio and sqrt(3) - 1 in 64-bit fixed point.
_PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
_PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def philox4x64(ctr, key, rounds: int = 10):
    """One Philox4x64 block: four 64-bit words from a 4-word counter and a 2-word key.
    Each round multiplies words 0 and 2 by the two constants, and the new words are
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key
    advances by the Weyl increments between rounds."""
    c0, c1, c2, c3 = (int(x) & _M64 for x in ctr)
    k0, k1 = (int(x) & _M64 for x in key)
    for _ in range(rounds):
        p0 = _PHILOX_M[0] * c0
        p1 = _PHILOX_M[1] * c2
        c0, c1, c2, c3 = (p1 >> 64) ^ c1 ^ k0, p1 & _M64, (p0 >> 64) ^ c3 ^ k1, p0 & _M64
        k0 = (k0 + _PHILOX_W[0]) & _M64
        k1 = (k1 + _PHILOX_W[1]) & _M64
    return [c0, c1, c2, c3]


def uniform(seed: int, counter: int, codebook: int) -> float:
    """The draw of (session seed, frame counter, codebook) in [0, 1), reading 7."""
    x = philox4x64((counter & 0xFFFFFFFF, codebook, 0, 0), (seed, 0))[0]
    return (x >> 40) * 2.0 ** -24


def process(logits, temperature: float, penalty: float = 1.0, seen=None):
    """Readings 2-3: the penalised, tempered scores z (float64) of a float32 row.
    NaN scores are excluded (-inf)."""
    x = np.asarray(logits, dtype=np.float64).copy()
    if seen is not None and penalty != 1.0:
        s = np.asarray(seen, dtype=bool)
        pos = s & (x > 0)
        neg = s & ~(x > 0)
        x[pos] = x[pos] / penalty
        x[neg] = x[neg] * penalty
    z = x / temperature
    z[np.isnan(z)] = -np.inf
    return z


def candidates(z, top_k: int):
    """Reading 4: indices of the top_k largest scores, ordered by (score descending,
    index ascending)."""
    order = sorted(range(len(z)), key=lambda i: (-z[i], i))
    return order[:max(1, min(top_k, len(z)))]


def sample(logits, u: float, temperature: float = 1.0, top_k: int = 50, top_p: float = 1.0,
           penalty: float = 1.0, seen=None):
    """Readings 2-6 for one row: returns (token, detail), where detail holds the
    candidate order, their cumulative weights, the kept count and the decision's
    distances to its boundaries (for telling ties from disagreements)."""
    z = process(logits, temperature, penalty, seen)
    cand = candidates(z, top_k)
    zc = np.array([z[i] for i in cand])
    if not np.isfinite(zc[0]):
        return cand[0], {"cand": cand, "cum": None, "kept": 1, "u_gap": math.inf,
                         "p_gap": math.inf, "k_gap": math.inf}
    w = np.exp(zc - zc[0])
    cum = np.cumsum(w)
    total = cum[-1]
    kept = int(np.sum(cum < top_p * total)) + 1
    kept = min(kept, len(cand))
    r = u * cum[kept - 1]
    j = int(np.argmax(cum[:kept] > r)) if np.any(cum[:kept] > r) else kept - 1
    # distances of the decision to its boundaries, relative to the kept total
    edges = np.concatenate([[0.0], cum[:kept]])
    u_gap = float(np.min(np.abs(edges - r)) / cum[kept - 1])
    p_gap = float(np.min(np.abs(cum - top_p * total)) / total)
    k_gap = math.inf
    if len(cand) < len(z):
        rest = np.sort(np.array([z[i] for i in range(len(z)) if i not in set(cand)]))[::-1]
        k_gap = float(zc[-1] - rest[0])
    return cand[j], {"cand": cand, "cum": cum, "kept": kept, "u_gap": u_gap, "p_gap": p_gap,
                     "k_gap": k_gap}


def distribution(logits, temperature: float = 1.0, top_k: int = 50, top_p: float = 1.0,
                 penalty: float = 1.0, seen=None):
    """The probability of every index under readings 2-6 with u uniform on [0, 1)."""
    z = process(logits, temperature, penalty, seen)
    cand = candidates(z, top_k)
    zc = np.array([z[i] for i in cand])
    w = np.exp(zc - zc[0])
    cum = np.cumsum(w)
    kept = min(int(np.sum(cum < top_p * cum[-1])) + 1, len(cand))
    p = np.zeros(len(z))
    for j in range(kept):
        p[cand[j]] = w[j] / cum[kept - 1]
    return p
