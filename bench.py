#!/usr/bin/env python3
"""Throughput of the lockstep decode frame on one MI355X.

A step is one decode frame for every session of the workload: the 28-layer
Talker step, codec head + greedy codebook 0, the 2048->1024 projection and the
15 code-predictor steps, replayed from one captured HIP graph.  The headline
workload is the B=32 full frame (ragged Talker KV 512..2048 positions in
16-token pages, 25 consecutive frames per sequence, bf16 weights); B=1 and
B=6 frames are reported beside it.  Inputs are seeded synthetic tensors, already
resident in device memory when the timed region starts.

Prints one JSON line (rank 0).  `value` is codec frames per second (one codec
frame = 16 codebook tokens for one session).
"""
import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix peak, published

# HBM bytes per launch of a kernel, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by 1 GiB / the same
# counter's reading for calibration_copy().  Keyed by (workload, kernel symbol), with
# the digest of the kernel sources the counters were taken on: once the kernels
# change, the entry no longer applies and `traffic` is reported as null.
PMC_TRAFFIC = {
    # profiles/gemm_attention_C4_pmc_traffic.md
    ("C4", "k_attn_paged"): {"digest": "09285f1884fd95bb", "bytes_per_launch": 164666749},
}
KERNEL_SOURCES = ["qt_gemm.hip", "qt_kernels.hip", "qt_device.h", "qt_internal.h"]


def kernel_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "streaming_tts_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(workload: str, kernel: str):
    e = PMC_TRAFFIC.get((workload, kernel))
    if e is None or e["digest"] != kernel_digest():
        return None
    return e["bytes_per_launch"]


def weight_bytes(d, int8: bool, distinct: bool = False, mode: str = "full") -> int:
    """Logical weight bytes one frame streams: every decode GEMM weight once per
    use for the whole batch (predictor layers once per predictor step).  With
    distinct=True, every matrix once per frame: the predictor's layers, which all
    15 steps share, are counted once (the stricter lower bound).
    mode "talker": the Talker layers, its final gain and the codec head only;
    mode "predictor": the projection and the predictor steps only."""
    def mat(n, k, narrow=True):
        # INT8 mode: int8 values + f32 row scales for the Talker's matrices, the
        # same values held as halves for the code predictor's (cache-resident)
        if not int8:
            return 2 * n * k
        return (n * k if narrow else 2 * n * k) + 4 * n

    def layer(x, narrow=True):
        return (mat(x.q_dim + 2 * x.kv_dim, x.hidden, narrow) + mat(x.hidden, x.q_dim, narrow)
                + mat(2 * x.ffn, x.hidden, narrow) + mat(x.hidden, x.ffn, narrow)
                + 2 * (2 * x.hidden + 2 * x.head_dim))
    t, p = d.talker, d.predictor
    head_rows = {"full": d.talker_vocab + p.hidden, "talker": d.talker_vocab,
                 "predictor": p.hidden}[mode]
    total = mat(head_rows, t.hidden)  # codec head and / or projection rows
    if mode != "predictor":
        total += t.layers * layer(t) + 2 * t.hidden
    if mode != "talker":
        pred_layers = p.layers * layer(p, narrow=False)
        pred_own = mat(d.code_vocab, p.hidden, narrow=False) + 2 * p.hidden  # each step's head, final gain
        total += (1 if distinct else d.n_steps) * pred_layers + d.n_steps * pred_own
    return total


def frame_bytes(d, lengths, int8: bool, distinct: bool = False, mode: str = "full") -> int:
    """Algorithmic bytes of one frame: weights (above) plus, per session, the
    Talker K/V read over positions 0..L (L = cached length before the frame), the
    appended K/V, the embedding rows, the input and the fp32 logits and tokens."""
    t = d.talker
    kv_pos = t.layers * t.n_kv * t.head_dim * 2 * 2  # K and V, bf16, all layers
    per_sess = 0
    for L in lengths:
        per_sess += 4 * d.n_codebooks + t.hidden * 2  # tokens; Talker input or h_in
        if mode != "predictor":
            per_sess += kv_pos * (int(L) + 1) + kv_pos + 4 * d.talker_vocab
        if mode != "talker":
            per_sess += d.n_steps * (d.predictor.hidden * 2 + 4 * d.code_vocab)
    return weight_bytes(d, int8, distinct, mode) + per_sess


def launch_bytes(d, kind, li, lengths, int8: bool) -> int:
    """Algorithmic bytes of one kernel launch of a frame whose sessions hold
    `lengths` cached Talker positions.
      GEMM:        the weight [n, k] once (bf16: 2nk; INT8: nk + 4n of row scales, or
                   2nk + 4n where the quantised values are held as halves), plus
                   the f32 logits a head writes (4 * m * n_logits); activations are
                   not counted (they could stay on chip).
      attn_paged:  per session, this layer's K and V over positions 0..L_b (the cache
                   plus the new one) and the appended pair: 4 * n_kv * head_dim * (L_b + 2).
      embed:       one bf16 embedding row per session.
      predictor:   the one-launch predictor: every step's layer and head weights, and per
                   session its embedding rows and f32 logits.
      others:      0 (predictor K/V is frame-local and could stay on chip)."""
    if kind == "gemm":
        w = {0: 2 * li.n * li.k, 1: li.n * li.k + 4 * li.n, 2: 2 * li.n * li.k + 4 * li.n}[li.int8]
        return w + 4 * li.m * li.n_logits
    if kind == "attn_paged":
        t = d.talker
        return int(sum(4 * t.n_kv * t.head_dim * (int(L) + 2) for L in lengths))
    if kind == "embed":
        return li.m * d.predictor.hidden * 2
    if kind == "predictor":  # every predictor step in one launch: layers and heads per step,
        p = d.predictor      # each session's embedding rows and logits
        proj = (p.hidden * d.talker.hidden + 4 * p.hidden) if int8 else 2 * p.hidden * d.talker.hidden
        return (weight_bytes(d, int8, mode="predictor") - proj
                + li.m * d.n_steps * (p.hidden * 2 + 4 * d.code_vocab))
    return 0


def trace_frames(dec, d, lengths, n, int8, log):
    """Run n frames whose every kernel carries start/stop events stamped with its
    own begin and end; aggregate by kernel symbol: launches, summed milliseconds,
    summed algorithmic bytes."""
    per = {}
    for f in range(n):
        for name, kind, li, ms in dec.trace("full", forced=False):
            e = per.setdefault(name, {"kind": kind, "launches": 0, "ms": 0.0, "bytes": 0})
            e["launches"] += 1
            e["ms"] += ms
            e["bytes"] += launch_bytes(d, kind, li, lengths + f, int8)
    total = sum(e["ms"] for e in per.values())
    for name, e in sorted(per.items(), key=lambda kv: -kv[1]["ms"]):
        e["avg_us"] = 1e3 * e["ms"] / e["launches"]
        e["gbs"] = e["bytes"] / (e["ms"] / 1e3) / 1e9
        e["share"] = e["ms"] / total
        log(f"[trace] {name:28s} {e['launches'] / n:6.0f}/frame {e['avg_us']:9.2f} us "
            f"{e['gbs']:8.1f} GB/s {100 * e['share']:5.1f}%")
    return per, total / n


def run_scheduler(pm, w, dec, lengths, steps, warmup, log):
    """The same workload decoded through the library's lockstep scheduler
    (qt_sched.h): every session submits its Talker input row and one qt_sched_step
    per frame decodes them all (captured sizes 1..32, so B=32 is one call).  The
    prefilled caches are copied device to device from `dec`'s pages into the pages
    the scheduler hands out.  GPU time is taken with events on the scheduler's
    stream around `steps` frames; host time is the loop's wall clock per frame."""
    import numpy as np
    import torch

    import synth
    from streaming_tts_decode_amd.runtime import PAGE, Scheduler
    frames = steps + warmup
    max_pages = int(max(-(-(int(L) + frames + 1) // PAGE) for L in lengths))
    sch = Scheduler(pm, buckets=(1, 2, 4, 8, 16, 32), max_sessions=w.batch, max_pages=max_pages,
                    num_pages=w.batch * max_pages + 1)
    sids = [sch.open(int(lengths[b]), copy_from=(dec.k_pages, dec.v_pages, dec.page_table_np[b]))
            for b in range(w.batch)]
    ins = synth.frame_inputs(w)["talker_in"]
    talker_all = torch.from_numpy(ins.view(np.int16)).to(dec.dev)
    for f in range(warmup):
        for b, sid in enumerate(sids):
            sch.submit(sid, talker_all[f % w.frames, b])
        sch.step()
    torch.cuda.synchronize()
    stream = sch.stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    t0 = time.perf_counter()
    groups = 0
    for f in range(steps):
        for b, sid in enumerate(sids):
            sch.submit(sid, talker_all[(warmup + f) % w.frames, b])
        groups += sch.step()
    host = time.perf_counter() - t0
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    status = sch.status()
    if status:
        raise RuntimeError(f"scheduler {w.name}: device status {status:#x}")
    sch.close()
    res = {"codec_frames_per_s": w.batch * steps / (ms / 1e3), "ms_per_frame": ms / steps,
           "host_ms_per_frame": 1e3 * host / steps, "calls_per_step": groups / steps,
           "pages": "handed out by the scheduler's free list: consecutive in a fresh pool "
                    "(the headline frame uses a shuffled pool)"}
    log(f"[bench] scheduler {w.name}: {res}")
    return res


def prefill_flops(d, lengths) -> float:
    """Multiply-adds x 2 of a prefill: every Talker projection for every row, causal
    attention (q.k and p.v over positions 0..p for each row), the codec head at each
    sequence's last row."""
    t = d.talker
    per_row = 2 * t.layers * ((t.q_dim + 2 * t.kv_dim) * t.hidden + t.hidden * t.q_dim
                              + 2 * t.ffn * t.hidden + t.hidden * t.ffn)
    flops = 0.0
    for L in lengths:
        flops += L * per_row + 2 * d.talker_vocab * t.hidden
        flops += t.layers * 4.0 * t.head_dim * t.n_q * L * (L + 1) / 2
    return flops


def run_prefill(pm, d, log, rows=1024, packings=((1024,), (256, 256, 256, 256)), reps=10):
    """Prompt prefill from a graph captured for `rows` rows, per packing of prompts:
    milliseconds per call, prompt tokens per second and achieved TFLOP/s against the
    dense fp16 MFMA peak (the projections run as fp16 x fp16 with f32 accumulation)."""
    import numpy as np
    import torch

    import synth
    from streaming_tts_decode_amd.runtime import Decoder
    out = {}
    for packing in packings:
        S = len(packing)
        max_pages = max(-(-L // 16) for L in packing)
        dec = Decoder(pm, batch=S, max_pages=max_pages)
        dec.prefill_setup(rows)
        prompts = [synth.normal_bf16(f"bench.prefill.{S}.{i}", (L, d.talker.hidden))
                   for i, L in enumerate(packing)]
        dec.prefill_inputs(prompts)
        g = dec.prefill_capture()
        stream = torch.cuda.current_stream()
        for _ in range(2):
            dec.replay(g)
        dec.status.zero_()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            dec.replay(g)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        if int(dec.status.item()):
            raise RuntimeError(f"prefill: device status {int(dec.status.item()):#x}")
        fl = prefill_flops(d, packing)
        res = {"rows": rows, "sequences": list(packing), "ms": ms,
               "tokens_per_s": sum(packing) / (ms / 1e3), "tflops": fl / (ms / 1e3) / 1e12,
               "mfma_frac": fl / (ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFLOPS}
        log(f"[bench] prefill {res}")
        out["x".join(str(L) for L in packing)] = res
        dec.close()
        del dec
        torch.cuda.empty_cache()
    return out


def run_workload(pm, w, steps, warmup, log, n_trace=0, extras=False):
    import numpy as np
    import torch

    import synth
    from streaming_tts_decode_amd.runtime import setup_workload
    frames = max(w.frames, steps + warmup + n_trace)
    wcap = dataclasses.replace(w, frames=frames)
    dec, lengths = setup_workload(wcap, pm)
    fin = synth.frame_inputs(w)
    if w.mode == "predictor":  # the post-norm Talker hidden and codebook-0 token per frame
        h_all = torch.from_numpy(fin["h_in"].view(np.int16)).to(dec.dev)
        tok_all = torch.from_numpy(fin["tok0"]).to(dec.dev)

        def feed(f):
            dec.h_in.copy_(h_all[f % w.frames], non_blocking=True)
            dec.tok0_in.copy_(tok_all[f % w.frames], non_blocking=True)
    else:
        talker_all = torch.from_numpy(fin["talker_in"].view(np.int16)).to(dec.dev)  # [frames, B, H]

        def feed(f):
            dec.talker_in.copy_(talker_all[f % w.frames], non_blocking=True)
    g = dec.capture(w.mode, forced=False)
    L0 = dec.kv_len.clone()
    stream = torch.cuda.current_stream()
    for f in range(warmup):
        feed(f)
        dec.replay(g)
    torch.cuda.synchronize()
    dec.kv_len.copy_(L0)
    dec.status.zero_()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for f in range(steps):
        feed(f)
        dec.replay(g)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1)
    status = int(dec.status.item())
    if status:
        raise RuntimeError(f"{w.name}: device status {status:#x}")
    adv = 0 if w.mode == "predictor" else 1  # cached lengths advance once per frame
    nbytes = sum(frame_bytes(w.dims, lengths + adv * f, pm.int8, mode=w.mode) for f in range(steps))
    nbytes_distinct = sum(frame_bytes(w.dims, lengths + adv * f, pm.int8, distinct=True, mode=w.mode)
                          for f in range(steps))
    per, traced_ms = (trace_frames(dec, w.dims, lengths + steps, n_trace, pm.int8, log)
                      if n_trace else (None, None))
    # repeated sequences (outside the timed region above): the workload's own frame
    # count from the same starting lengths, each timed alone; min and median
    seq_ms = []
    for rep in range(5 if extras else 0):
        dec.kv_len.copy_(L0)
        torch.cuda.synchronize()
        ev0.record(stream)
        for f in range(w.frames):
            dec.talker_in.copy_(talker_all[f % w.frames], non_blocking=True)
            dec.replay(g)
        ev1.record(stream)
        torch.cuda.synchronize()
        seq_ms.append(ev0.elapsed_time(ev1) / w.frames)
    if int(dec.status.item()):
        raise RuntimeError(f"{w.name} sequences: device status {int(dec.status.item()):#x}")
    sequences = ({"reps": len(seq_ms), "frames": w.frames, "min_ms_per_frame": min(seq_ms),
                  "median_ms_per_frame": float(np.median(seq_ms)),
                  "max_codec_frames_per_s": w.batch / (min(seq_ms) / 1e3)} if seq_ms else None)
    sampled = None
    if extras:
        # the same frames drawing every codebook (qt_sampling) instead of the argmax
        dec.set_sampling((0.9, 1.0, 1.05, 50), (0.9, 1.0, 1.0, 50), list(range(1, w.batch + 1)))
        gs = dec.capture("full", forced=False, sampling=True)
        for f in range(warmup):
            dec.talker_in.copy_(talker_all[f % w.frames], non_blocking=True)
            dec.replay(gs)
        dec.kv_len.copy_(L0)
        dec.status.zero_()
        torch.cuda.synchronize()
        ev0.record(stream)
        for f in range(steps):
            dec.talker_in.copy_(talker_all[f % w.frames], non_blocking=True)
            dec.replay(gs)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_s = ev0.elapsed_time(ev1)
        if int(dec.status.item()):
            raise RuntimeError(f"{w.name} sampled: device status {int(dec.status.item()):#x}")
        sampled = {"codec_frames_per_s": w.batch * steps / (ms_s / 1e3), "ms_per_frame": ms_s / steps,
                   "vs_greedy": ms / ms_s,
                   "params": "codebook 0: T 0.9, top_k 50, top_p 1.0, penalty 1.05; "
                             "predictor: T 0.9, top_k 50, top_p 1.0"}
        log(f"[bench] sampled {w.name}: {sampled}")
    res = {
        "workload": w.name, "batch": w.batch, "frames": steps,
        "ms_per_frame": ms / steps, "codec_frames_per_s": w.batch * steps / (ms / 1e3),
        "hbm_gbs_algorithmic": nbytes / (ms / 1e3) / 1e9,
        "bytes_per_frame": nbytes / steps, "wall_s": wall,
        "kernels": per, "traced_ms_per_frame": traced_ms, "sampled": sampled, "sequences": sequences,
    }
    res["hbm_frac"] = res["hbm_gbs_algorithmic"] / HBM_PEAK_GBS
    # the stricter figure: each matrix once per frame (the shared predictor layers once)
    res["hbm_frac_distinct"] = nbytes_distinct / (ms / 1e3) / 1e9 / HBM_PEAK_GBS
    log(f"[bench] { {k: v for k, v in res.items() if k != 'kernels'} }")
    dec.close()
    if extras:
        s = run_scheduler(pm, w, dec, lengths, steps, warmup, log)
        s["vs_graph"] = s["codec_frames_per_s"] / res["codec_frames_per_s"]
        res["scheduler"] = s
    del dec
    torch.cuda.empty_cache()
    return res, lengths


def roofline(res, n_trace):
    """The kernel symbol with the largest share of the traced frames' time, against
    the HBM roofline: algorithmic bytes per launch / average launch duration."""
    per = res["kernels"]
    name = max(per, key=lambda k: per[k]["ms"])
    e = per[name]
    return {
        "bound": "hbm", "kernel": name,
        "achieved": e["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": e["gbs"] / HBM_PEAK_GBS,
        "traffic": pmc_traffic(res["workload"], name),
        "avg_launch_us": e["avg_us"], "launches_per_frame": e["launches"] / n_trace,
        "algorithmic_bytes_per_launch": e["bytes"] / e["launches"],
        "share_of_frame": e["share"],
        "timing": f"start/stop HIP events stamped by each kernel (hipExtLaunchKernel) over "
                  f"{n_trace} frames on the frame's stream",
    }


def calibration_copy(log):
    """A plain 1 GiB device-to-device copy: the byte count hardware counters read for
    it calibrates their readings of the decode kernels."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[calib] copied {n} bytes device to device")
    del src, dst


def host_cpu() -> dict:
    """The host's CPU model name (first "model name" of /proc/cpuinfo), the logical
    CPUs it has and the ones this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def cpu_baseline(w, weights, seconds: float, log):
    """The oracle, as it stands, on the host cores, compiled for this host
    (gcc -O3 -march=native -fopenmp, no fast-math or contraction: the same results
    as the portable build the tests use):
      * session 0 of the workload, consecutive full frames until `seconds` of
        wall time have run, with every OpenMP thread (the headline baseline);
      * on one thread: one predictor-only frame (the C1 workload) and one Talker
        step over 256 cached positions (the C2 workload), the per-core rates."""
    import oracle
    import synth
    flags = oracle.use_native_build()
    threads = oracle.max_threads()
    d = w.dims
    t = d.talker
    orc = oracle.OracleModel(d, weights, int8=w.int8)
    L = int(w.lengths()[0])
    kb, vb = synth.gen_kv(w.name, 0, t.layers, L, t.n_kv, t.head_dim)
    ins = synth.frame_inputs(w)["talker_in"][:, 0]
    kc, vc = orc.new_cache(L + w.frames, kb, vb)
    n, length = 0, L
    t0 = time.perf_counter()
    while n < w.frames and (n == 0 or time.perf_counter() - t0 < seconds):
        _, length = orc.frame("full", kc, vc, length, talker_in=oracle.bf16_to_f64(ins[n]))
        n += 1
    el = time.perf_counter() - t0
    one = {}
    oracle.set_threads(1)
    try:
        c1 = synth.WORKLOADS["C1"]
        f1 = synth.frame_inputs(c1)
        t1 = time.perf_counter()
        orc.frame("predictor", h_in=oracle.bf16_to_f64(f1["h_in"][0, 0]), tok0=int(f1["tok0"][0, 0]))
        one["C1_predictor_frames_per_s"] = 1.0 / (time.perf_counter() - t1)
        c2 = synth.WORKLOADS["C2"]
        L2 = int(c2.lengths()[0])
        kb2, vb2 = synth.gen_kv(c2.name, 0, t.layers, L2, t.n_kv, t.head_dim)
        kc2, vc2 = orc.new_cache(L2 + 1, kb2, vb2)
        x2 = synth.frame_inputs(c2)["talker_in"][0, 0]
        t2 = time.perf_counter()
        orc.frame("talker", kc2, vc2, L2, talker_in=oracle.bf16_to_f64(x2))
        one["C2_talker_steps_per_s"] = 1.0 / (time.perf_counter() - t2)
    finally:
        oracle.set_threads(threads)
    res = {"value": n / el, "unit": "codec frames/s", "cores": threads, "kind": "oracle",
           "sample": f"{w.name} session 0 (L={L}), {n} consecutive full frames on {threads} "
                     f"threads, float64 C oracle, {el:.1f} s",
           "threads": threads, **host_cpu(), "compiler": "gcc " + " ".join(flags),
           "one_thread": one}
    log(f"[cpu] {res}")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=25)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C4")
    ap.add_argument("--also", default="B1,C3", help="extra workloads reported beside the headline")
    ap.add_argument("--parts", default="C1,C2",
                    help="the predictor-only frame and the Talker step, timed on their own")
    ap.add_argument("--int8", action="store_true", help="INT8 weight-only decode")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-int8", action="store_true",
                    help="skip timing the INT8 weight-only frames (C4, B=1)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip timing the prompt prefill (1024 rows)")
    ap.add_argument("--no-scheduler", action="store_true",
                    help="skip the headline workload's extra timings: through the lockstep "
                         "scheduler, with every codebook drawn, and as repeated sequences")
    ap.add_argument("--trace-frames", type=int, default=5,
                    help="eager frames timed launch by launch for the roofline")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: runs on exactly one GPU (sessions would shard across GPUs with no "
              "communication; runs on several GPUs are not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import streaming_tts_decode_amd as qt
    import synth
    from streaming_tts_decode_amd.runtime import PackedModel

    qt.lib()  # fails loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    head = synth.WORKLOADS[args.workload]
    if args.int8:
        head = dataclasses.replace(head, int8=True)
    d = head.dims
    log(f"[bench] kernel sources digest {kernel_digest()}")
    log(f"[bench] generating weights")
    W = synth.gen_weights(d)
    pm = PackedModel(d, W, int8=head.int8)
    main_res, lengths = run_workload(pm, head, args.steps, args.warmup, log,
                                     n_trace=max(1, args.trace_frames),
                                     extras=not args.no_scheduler)
    extra = {}
    for name in [x for x in args.also.split(",") if x]:
        w = dataclasses.replace(synth.WORKLOADS[name], int8=head.int8)
        r, _ = run_workload(pm, w, args.steps, args.warmup, log)
        extra[f"B{w.batch}"] = {k: r[k] for k in ("codec_frames_per_s", "ms_per_frame",
                                                  "hbm_gbs_algorithmic", "hbm_frac", "hbm_frac_distinct")}
    # the predictor-only frame (C1) and the Talker step (C2), each at B = 1 from its
    # own graph: frames (or Talker steps) per second and their algorithmic HBM rate
    parts = {}
    for name in [x for x in args.parts.split(",") if x]:
        w = dataclasses.replace(synth.WORKLOADS[name], int8=head.int8)
        r, _ = run_workload(pm, w, args.steps, args.warmup, log)
        unit = "Talker steps/s" if w.mode == "talker" else "predictor frames/s"
        parts[name] = {"note": w.note, "per_s": r["codec_frames_per_s"], "unit": unit,
                       "ms_per_call": r["ms_per_frame"], "bytes_per_call": r["bytes_per_frame"],
                       "hbm_gbs_algorithmic": r["hbm_gbs_algorithmic"], "hbm_frac": r["hbm_frac"],
                       "hbm_frac_distinct": r["hbm_frac_distinct"]}
    prefill = None if args.no_prefill else run_prefill(pm, d, log)
    pm.close()
    int8 = None
    if not args.int8 and not args.no_int8:
        # the INT8 weight-only frame (quantized at load from the same bf16 tensors)
        pm8 = PackedModel(d, W, int8=True)
        int8 = {}
        for name in ("C4", "B1"):
            w = dataclasses.replace(synth.WORKLOADS[name], int8=True)
            r, _ = run_workload(pm8, w, args.steps, args.warmup, log)
            int8[name] = {k: r[k] for k in ("codec_frames_per_s", "ms_per_frame",
                                             "hbm_gbs_algorithmic", "hbm_frac", "hbm_frac_distinct",
                                             "bytes_per_frame")}
        pm8.close()
    calibration_copy(log)
    cpu = None if args.no_cpu_baseline else cpu_baseline(head, W, args.cpu_seconds, log)

    out = {
        "metric": "codec frames/sec (Talker step + 15 code-predictor steps per session frame)",
        "value": main_res["codec_frames_per_s"],
        "unit": "codec frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_frame"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int8 source weights quantized per row, fp16 operands, fp32 accumulate"
                  if head.int8 else "bf16 source weights, fp16 operands, fp32 accumulate"),
        "data": "synthetic: seeded N(0,0.02) bf16 weights, N(0,1) inputs and prefilled KV",
        "config": {"workload": f"{head.name}: {head.note}", "batch": head.batch,
                   "kv_len": f"{head.len_lo}..{head.len_hi} (ragged, 16-token pages)",
                   "frames_per_sequence": head.frames, "graph": True,
                   "parallelism": "single GPU"},
        "frame_hbm_gbs": main_res["hbm_gbs_algorithmic"],
        "frame_hbm_frac": main_res["hbm_frac"],
        "frame_hbm_frac_distinct": main_res["hbm_frac_distinct"],
        "bytes_per_frame": main_res["bytes_per_frame"],
        "other_batches": extra,
        "parts": parts,
        "scheduler": main_res.get("scheduler"),
        "sampled": main_res.get("sampled"),
        "sequences": main_res.get("sequences"),
        "prefill": prefill,
        "int8": int8,
        "roofline": roofline(main_res, max(1, args.trace_frames)),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
