"""Seeded synthetic inputs for the lockstep decode frame.

This module is the only code that both the CPU oracle and the HIP path see.
It draws random numbers and lays them out; it holds none of the decode
arithmetic (no norm, no rotation, no attention, no projection).

Recipe
------
* Base seed 20261202.  Every tensor gets its own stream:
  ``PCG64(SeedSequence(seed, spawn_key=(crc32(name), chunk)))`` where large
  tensors are cut into fixed chunks of ``CHUNK`` values so that chunks can be
  drawn in parallel threads and adding a tensor never shifts another.
* Normal samples are drawn in float32 and rounded to bfloat16 with
  round-to-nearest-even (torch's CPU conversion).
* Weights: N(0, 0.02).  Norm gains: exactly 1.0 unless ``gain_std`` > 0, in
  which case N(1, gain_std) (used by the small oracle pins, because gains of
  1.0 hide a swapped-gain mistake).
* Talker input hidden states, predictor input hidden states and prefilled K/V
  contents: N(0, 1).
* Per-session KV lengths: integers uniform on [lo, hi], both ends included.
* Codebook-0 tokens for the predictor-only workload: uniform on [0, 2048).

The model dimensions follow the workload descriptions of the Qwen3-TTS
12 Hz 1.7B decode frame on the pages ("Qwen3-TTS Native v0.3.0", What
changed; the M* "Qwen3-TTS PR 5" page, What changed vs the 0.6B port: the
2048 -> 1024 projection; the decomputer.nl article, section 3: 15 fixed
code-predictor steps).
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

BASE_SEED = 20261202
CHUNK = 1 << 22  # values per independently seeded chunk


# --------------------------------------------------------------------------
# dimensions
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class DecoderDims:
    layers: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    rope_theta: float = 1.0e6
    eps: float = 1.0e-6

    @property
    def q_dim(self) -> int:
        return self.n_q * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv * self.head_dim


@dataclass(frozen=True)
class ModelDims:
    talker: DecoderDims
    predictor: DecoderDims
    talker_vocab: int = 3072
    code_vocab: int = 2048
    cb0_range: int = 2048     # codebook-0 argmax runs over [0, cb0_range)
    n_codebooks: int = 16     # 1 Talker codebook + (n_codebooks - 1) predictor steps
    page_size: int = 16

    @property
    def n_steps(self) -> int:
        return self.n_codebooks - 1


FULL = ModelDims(
    talker=DecoderDims(layers=28, hidden=2048, n_q=16, n_kv=8, head_dim=128, ffn=6144),
    predictor=DecoderDims(layers=5, hidden=1024, n_q=16, n_kv=8, head_dim=128, ffn=3072),
)

# A reduced model with the same head geometry (head_dim 128, 2 query heads per
# KV head) that the GPU path accepts; used for fast GPU edge-case tests.
SMALL = ModelDims(
    talker=DecoderDims(layers=2, hidden=1024, n_q=8, n_kv=4, head_dim=128, ffn=1536),
    predictor=DecoderDims(layers=2, hidden=512, n_q=8, n_kv=4, head_dim=128, ffn=1024),
    talker_vocab=1536, code_vocab=1024, cb0_range=1024, n_codebooks=5, page_size=16,
)

# A tiny model for oracle-only pins (brute force in float64 NumPy).
TINY = ModelDims(
    talker=DecoderDims(layers=2, hidden=64, n_q=4, n_kv=2, head_dim=16, ffn=96),
    predictor=DecoderDims(layers=2, hidden=32, n_q=4, n_kv=2, head_dim=16, ffn=48),
    talker_vocab=40, code_vocab=32, cb0_range=32, n_codebooks=4, page_size=4,
)


# --------------------------------------------------------------------------
# tensor table
# --------------------------------------------------------------------------
GAIN, WEIGHT, EMBED = "gain", "weight", "embed"


def _layer_specs(prefix: str, d: DecoderDims):
    out = []
    for l in range(d.layers):
        p = f"{prefix}.layers.{l}."
        out += [
            (p + "input_norm", (d.hidden,), GAIN),
            (p + "q_proj", (d.q_dim, d.hidden), WEIGHT),
            (p + "k_proj", (d.kv_dim, d.hidden), WEIGHT),
            (p + "v_proj", (d.kv_dim, d.hidden), WEIGHT),
            (p + "q_norm", (d.head_dim,), GAIN),
            (p + "k_norm", (d.head_dim,), GAIN),
            (p + "o_proj", (d.hidden, d.q_dim), WEIGHT),
            (p + "post_norm", (d.hidden,), GAIN),
            (p + "gate_proj", (d.ffn, d.hidden), WEIGHT),
            (p + "up_proj", (d.ffn, d.hidden), WEIGHT),
            (p + "down_proj", (d.hidden, d.ffn), WEIGHT),
        ]
    out.append((prefix + ".final_norm", (d.hidden,), GAIN))
    return out


def tensor_specs(m: ModelDims):
    """(name, shape, kind) for every weight tensor of the model, in a fixed order."""
    t, p = m.talker, m.predictor
    specs = _layer_specs("talker", t)
    specs.append(("talker.codec_head", (m.talker_vocab, t.hidden), WEIGHT))
    specs.append(("projection", (p.hidden, t.hidden), WEIGHT))
    specs += _layer_specs("predictor", p)
    for i in range(m.n_steps):
        specs.append((f"predictor.codec_embed.{i}", (m.code_vocab, p.hidden), EMBED))
        specs.append((f"predictor.lm_head.{i}", (m.code_vocab, p.hidden), WEIGHT))
    return specs


def linear_names(m: ModelDims):
    """Names of every decode GEMM weight (the ones INT8 mode quantizes)."""
    return [n for n, _, k in tensor_specs(m) if k == WEIGHT]


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------
def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _stream(name: str, chunk: int, seed: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(zlib.crc32(name.encode()), chunk))
    return np.random.Generator(np.random.PCG64(ss))


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(name: str, n: int, mean: float, std: float, seed: int = BASE_SEED,
               pool: ThreadPoolExecutor | None = None) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        _stream(name, c, seed).standard_normal(dtype=np.float32, out=out[lo:hi])

    if pool is not None and nchunks > 1:
        list(pool.map(fill, range(nchunks)))
    else:
        for c in range(nchunks):
            fill(c)
    if std != 1.0:
        out *= np.float32(std)
    if mean != 0.0:
        out += np.float32(mean)
    return out


def normal_bf16(name: str, shape, mean: float = 0.0, std: float = 1.0,
                seed: int = BASE_SEED, pool=None) -> np.ndarray:
    n = int(np.prod(shape))
    return _to_bf16_bits(normal_f32(name, n, mean, std, seed, pool)).reshape(shape)


def gen_weights(m: ModelDims, seed: int = BASE_SEED, gain_std: float = 0.0,
                weight_std: float = 0.02, embed_std: float = 0.02) -> dict:
    """All model tensors as bfloat16 bit patterns (np.uint16), keyed by name."""
    specs = tensor_specs(m)
    out = {}
    with ThreadPoolExecutor(_threads()) as pool:
        def one(spec):
            name, shape, kind = spec
            if kind == GAIN:
                if gain_std == 0.0:
                    return name, np.full(shape, 0x3F80, dtype=np.uint16)  # 1.0
                return name, normal_bf16(name, shape, 1.0, gain_std, seed)
            std = weight_std if kind == WEIGHT else embed_std
            return name, normal_bf16(name, shape, 0.0, std, seed)
        for name, arr in pool.map(one, specs):
            out[name] = arr
    return out


def uniform_ints(name: str, n: int, lo: int, hi: int, seed: int = BASE_SEED) -> np.ndarray:
    """n integers uniform on [lo, hi] (both ends included)."""
    return _stream(name, 0, seed).integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.int32)


def gen_kv(tag: str, session: int, layers: int, length: int, n_kv: int, head_dim: int,
           seed: int = BASE_SEED, pool=None):
    """Prefilled Talker cache contents for one session: K and V, each
    [layers, length, n_kv, head_dim] bfloat16 bits, N(0, 1)."""
    shape = (layers, length, n_kv, head_dim)
    k = normal_bf16(f"{tag}.kv.k.s{session}", shape, 0.0, 1.0, seed, pool)
    v = normal_bf16(f"{tag}.kv.v.s{session}", shape, 0.0, 1.0, seed, pool)
    return k, v


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    mode: str              # "full" | "talker" | "predictor"
    batch: int
    frames: int
    len_lo: int = 0        # Talker KV length range (inclusive)
    len_hi: int = 0
    int8: bool = False
    graph: bool = False
    dims: ModelDims = field(default=FULL)
    note: str = ""
    lens: tuple = ()       # explicit per-session lengths (overrides the range)

    def lengths(self, seed: int = BASE_SEED) -> np.ndarray:
        if self.mode == "predictor":
            return np.zeros(self.batch, dtype=np.int32)
        if self.lens:
            return np.asarray(self.lens, dtype=np.int32)
        if self.len_lo == self.len_hi:
            return np.full(self.batch, self.len_lo, dtype=np.int32)
        return uniform_ints(f"{self.name}.kv_len", self.batch, self.len_lo, self.len_hi, seed)

    def max_pages(self) -> int:
        ps = self.dims.page_size
        return max(1, -(-(int(self.lengths().max()) + self.frames) // ps))


WORKLOADS = {
    "C1": Workload("C1", "predictor", batch=1, frames=1,
                   note="CodePredictor-only frame, 1 session"),
    "C2": Workload("C2", "talker", batch=1, frames=1, len_lo=256, len_hi=256,
                   note="Talker single decode step, 1 session, 256 prefilled positions"),
    "C3": Workload("C3", "full", batch=6, frames=12, len_lo=64, len_hi=512,
                   note="full lockstep frame, B=6, bf16, 12 teacher-forced frames"),
    "C4": Workload("C4", "full", batch=32, frames=25, len_lo=512, len_hi=2048, graph=True,
                   note="full lockstep frame, B=32, bf16, 25 frames replayed from one graph"),
    "C5B1": Workload("C5B1", "full", batch=1, frames=25, len_lo=512, len_hi=2048, int8=True,
                     graph=True, note="INT8 weight-only decode, B=1, otherwise as C4"),
    "C5B32": Workload("C5B32", "full", batch=32, frames=25, len_lo=512, len_hi=2048, int8=True,
                      graph=True, note="INT8 weight-only decode, B=32, otherwise as C4"),
    "B1": Workload("B1", "full", batch=1, frames=25, len_lo=512, len_hi=2048, graph=True,
                   note="full lockstep frame, B=1, bf16, C4 settings"),
}


def frame_inputs(w: Workload, seed: int = BASE_SEED):
    """Per-frame inputs.  Returns a dict with
    talker_in [frames, B, Ht] bf16 bits (full / talker modes),
    h_in [frames, B, Ht] bf16 bits and tok0 [frames, B] int32 (predictor mode)."""
    d = w.dims
    out = {}
    if w.mode in ("full", "talker"):
        out["talker_in"] = normal_bf16(f"{w.name}.talker_in", (w.frames, w.batch, d.talker.hidden))
    else:
        out["h_in"] = normal_bf16(f"{w.name}.h_in", (w.frames, w.batch, d.talker.hidden))
        out["tok0"] = uniform_ints(f"{w.name}.tok0", w.frames * w.batch, 0, d.cb0_range - 1,
                                   seed).reshape(w.frames, w.batch)
    return out


def with_dims(w: Workload, dims: ModelDims, **kw) -> Workload:
    return replace(w, dims=dims, **kw)
