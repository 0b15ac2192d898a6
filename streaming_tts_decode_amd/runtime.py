"""Device-memory plumbing around the C ABI, with PyTorch as the allocator.

`Decoder` owns every buffer one qt_frame_decode call needs: the packed
weights, the workspace, the Talker KV page pools and page tables, and the
input/output tensors.  It lays prefilled per-session caches out into pages and
fills descriptors; all decoding happens inside libqt.so.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import (KERNEL_KINDS, FrameInputs, FrameOutputs, KvCaches, MODES, QT_BF16, PrefillArgs,
               Sampling, Sessions, qt_prefill, qt_prefill_graph_create, qt_prefill_workspace_bytes,
               make_cfg, make_sched_cfg, qt_frame_decode, qt_frame_decode_noalloc,
               qt_frame_graph_create,
               qt_frame_graph_launch, qt_frame_launch_count, qt_frame_trace, qt_graph_destroy,
               qt_load_weights, qt_model_destroy, qt_packed_bytes, qt_sched_bytes, qt_sched_close,
               qt_sched_create, qt_sched_destroy, qt_sched_free_pages, qt_sched_length,
               qt_sched_set_sampling,
               qt_sched_open, qt_sched_outputs, qt_sched_state, qt_sched_status_word,
               qt_sched_step, qt_sched_submit, qt_trace_create, qt_trace_destroy, qt_trace_read,
               qt_workspace_bytes)

PAGE = 16


def _aligned(torch, nbytes: int, device, align: int = 256):
    buf = torch.empty(nbytes + align, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % align
    return buf, buf.data_ptr() + off


def _bits(torch, a: np.ndarray, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(device)


def _write_pages(torch, k_pool, v_pool, pages, k_bits: np.ndarray, v_bits: np.ndarray):
    """Store a prefilled cache ([layers, L, n_kv, hd] bf16 bits) into `pages` (page
    ids in position order) of the pools [layers][num_pages][n_kv][PAGE][hd]."""
    layers, L, nkv, hd = k_bits.shape
    npg = len(pages)
    if npg == 0:
        return
    dev = k_pool.device
    idx = torch.from_numpy(np.asarray(pages, dtype=np.int64)).to(dev)
    for src, pool in ((k_bits, k_pool), (v_bits, v_pool)):
        x = np.zeros((layers, npg * PAGE, nkv, hd), dtype=np.uint16)
        x[:, :L] = src
        t = _bits(torch, x, dev).view(layers, npg, PAGE, nkv, hd).permute(0, 1, 3, 2, 4)
        pool[:, idx] = t


class PackedModel:
    """The model's weights packed by qt_load_weights into one device buffer.

    weights: name -> bfloat16 bits (np.uint16), as produced by synth.gen_weights."""

    def __init__(self, dims, weights: dict, int8: bool = False, device="cuda"):
        import torch
        self.torch = torch
        self.dims = dims
        self.dev = torch.device(device)
        self.cfg = make_cfg(dims)
        self.int8 = int8
        stream = torch.cuda.current_stream(self.dev)
        src, table = {}, []
        for name, arr in weights.items():
            t = _bits(torch, arr, self.dev)
            src[name] = t
            rows, cols = (1, arr.shape[0]) if arr.ndim == 1 else arr.shape
            table.append((name, t.data_ptr(), QT_BF16, int(rows), int(cols)))
        self.packed_bytes = qt_packed_bytes(self.cfg, int(int8))
        self._packed_buf, self.packed_ptr = _aligned(torch, self.packed_bytes, self.dev)
        self.handle = qt_load_weights(self.cfg, table, int(int8), self.packed_ptr,
                                      self.packed_bytes, stream.cuda_stream)
        torch.cuda.synchronize(self.dev)
        del src

    def close(self):
        if self.handle:
            qt_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Decoder:
    """Buffers for up to `batch` sessions of one PackedModel.

    max_pages: page-table row length (capacity = max_pages * 16 positions).
    num_pages: size of the shared page pool (default batch * max_pages)."""

    def __init__(self, model: PackedModel, batch: int = 1, max_pages: int = 1,
                 num_pages: int | None = None, page_seed: int = 1234):
        import torch
        self.torch = torch
        self.pm = model
        self.model = model.handle
        dims = model.dims
        self.dims = dims
        self.dev = model.dev
        self.B = batch
        self.max_pages = max_pages
        self.num_pages = num_pages if num_pages is not None else batch * max_pages
        self.cfg = model.cfg
        self.int8 = model.int8

        t, p = dims.talker, dims.predictor
        self.ws_bytes = qt_workspace_bytes(self.cfg, batch, max_pages)
        self._ws_buf, self.ws_ptr = _aligned(torch, self.ws_bytes, self.dev)
        shape = (t.layers, self.num_pages, t.n_kv, PAGE, t.head_dim)
        self.k_pages = torch.zeros(shape, dtype=torch.int16, device=self.dev)
        self.v_pages = torch.zeros(shape, dtype=torch.int16, device=self.dev)
        rng = np.random.default_rng(page_seed)
        perm = rng.permutation(self.num_pages).astype(np.int32)
        table_np = np.full((batch, max_pages), -1, dtype=np.int32)
        for b in range(batch):
            chunk = perm[b * max_pages:(b + 1) * max_pages]
            table_np[b, :len(chunk)] = chunk
        self.page_table_np = table_np
        self.page_table = torch.from_numpy(table_np).to(self.dev)
        self.kv_len = torch.zeros(batch, dtype=torch.int32, device=self.dev)

        self.talker_in = torch.zeros((batch, t.hidden), dtype=torch.int16, device=self.dev)
        self.h_in = torch.zeros((batch, t.hidden), dtype=torch.int16, device=self.dev)
        self.tok0_in = torch.zeros(batch, dtype=torch.int32, device=self.dev)
        self.forced = torch.zeros((batch, dims.n_codebooks), dtype=torch.int32, device=self.dev)
        self.logits0 = torch.zeros((batch, dims.talker_vocab), dtype=torch.float32, device=self.dev)
        self.logits_pred = torch.zeros((batch, dims.n_steps, dims.code_vocab), dtype=torch.float32,
                                       device=self.dev)
        self.tokens = torch.zeros((batch, dims.n_codebooks), dtype=torch.int32, device=self.dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=self.dev)
        # sampling state: [b][0] codebook-0 and [b][1] predictor parameters (16 bytes
        # each: temperature, top_p, repetition_penalty as f32, top_k as i32), seeds,
        # and the seen sets of codebook-0 tokens; the draw counter is kv_len
        self.sampler_params = torch.zeros((batch, 2, 4), dtype=torch.int32, device=self.dev)
        self.seed = torch.zeros(batch, dtype=torch.int64, device=self.dev)
        self.seen0 = torch.zeros((batch, (dims.cb0_range + 31) // 32), dtype=torch.int32,
                                 device=self.dev)
        self.graphs = []
        self._trace = None

    # ------------------------------------------------------------------ state
    def load_session_kv(self, b: int, k_bits: np.ndarray, v_bits: np.ndarray):
        """Lay a session's prefilled cache ([layers, L, n_kv, hd] bf16 bits) out
        into its pages and set kv_len[b] = L."""
        torch = self.torch
        layers, L, nkv, hd = k_bits.shape
        npg = -(-L // PAGE)
        if npg > self.max_pages:
            raise ValueError(f"session {b}: {L} positions need {npg} pages > {self.max_pages}")
        _write_pages(torch, self.k_pages, self.v_pages, self.page_table_np[b, :npg], k_bits, v_bits)
        self.kv_len[b] = L

    def set_lengths(self, lengths):
        self.kv_len.copy_(self.torch.as_tensor(np.asarray(lengths, dtype=np.int32)))

    def set_inputs(self, talker_in=None, h_in=None, tok0=None, forced=None):
        torch = self.torch
        if talker_in is not None:
            self.talker_in.copy_(_bits(torch, talker_in, self.dev))
        if h_in is not None:
            self.h_in.copy_(_bits(torch, h_in, self.dev))
        if tok0 is not None:
            self.tok0_in.copy_(torch.as_tensor(np.asarray(tok0, dtype=np.int32)))
        if forced is not None:
            self.forced.copy_(torch.as_tensor(np.asarray(forced, dtype=np.int32)))

    def set_sampling(self, talker, predictor, seeds):
        """talker / predictor: per-session (temperature, top_p, repetition_penalty,
        top_k) tuples (or one tuple for all); seeds: per-session integers."""
        def rows(p):
            p = list(p) if isinstance(p[0], (tuple, list)) else [p] * self.B
            return p
        rec = np.zeros((self.B, 2), dtype=[("t", "<f4"), ("p", "<f4"), ("r", "<f4"), ("k", "<i4")])
        for g, ps in enumerate((rows(talker), rows(predictor))):
            for b, (t, p, r, k) in enumerate(ps):
                rec[b, g] = (t, p, r, k)
        self.sampler_params.copy_(self.torch.from_numpy(rec.view(np.int32).reshape(self.B, 2, 4)))
        self.seed.copy_(self.torch.as_tensor(np.asarray(seeds, dtype=np.uint64).view(np.int64)))

    # ------------------------------------------------------------------ descriptors
    def _descs(self, mode: str, forced: bool, batch: int | None = None, sampling: bool = False,
               seen: bool = True):
        B = batch or self.B
        ss = Sessions(B, self.kv_len.data_ptr(), self.page_table.data_ptr(), self.max_pages)
        kv = KvCaches(self.k_pages.data_ptr(), self.v_pages.data_ptr(), self.num_pages)
        fi = FrameInputs(MODES[mode], self.talker_in.data_ptr(), self.h_in.data_ptr(),
                         self.tok0_in.data_ptr(), self.forced.data_ptr() if forced else None)
        if sampling:
            self._sampling = Sampling(self.sampler_params.data_ptr(), self.seed.data_ptr(),
                                      self.kv_len.data_ptr(),
                                      self.seen0.data_ptr() if seen else None)
            fi.sampling = C.pointer(self._sampling)
        fo = FrameOutputs(self.logits0.data_ptr(), self.logits_pred.data_ptr(),
                          self.tokens.data_ptr(), self.status.data_ptr())
        return ss, kv, fi, fo

    def decode(self, mode: str = "full", forced: bool = False, batch: int | None = None,
               sampling: bool = False, seen: bool = True):
        """Enqueue one frame on the current stream (no host synchronisation).  With
        sampling, tokens are drawn with the parameters of set_sampling and kv_len as
        the draw counter."""
        ss, kv, fi, fo = self._descs(mode, forced, batch, sampling, seen)
        qt_frame_decode(self.model, ss, kv, fi, fo, self.ws_ptr, self.ws_bytes,
                        self.torch.cuda.current_stream(self.dev).cuda_stream)

    def decode_noalloc(self, mode: str = "full", forced: bool = False, batch: int | None = None):
        """The same frame through qt_frame_decode_noalloc: the library's static
        scratch instead of this decoder's workspace."""
        ss, kv, fi, fo = self._descs(mode, forced, batch)
        qt_frame_decode_noalloc(self.model, ss, kv, fi, fo,
                                self.torch.cuda.current_stream(self.dev).cuda_stream)

    # ------------------------------------------------------------------ prompt prefill
    def prefill_setup(self, rows: int):
        """Buffers for prefills of up to `rows` packed rows into this decoder's
        sessions (sequence s = session s, its pages from the page table)."""
        torch, d = self.torch, self.dims
        self.pf_rows = rows
        self.pf_ws_bytes = qt_prefill_workspace_bytes(self.cfg, rows, self.B)
        self._pf_ws_buf, self.pf_ws_ptr = _aligned(torch, self.pf_ws_bytes, self.dev)
        self.pf_seq_start = torch.zeros(self.B + 1, dtype=torch.int32, device=self.dev)
        self.pf_embeds = torch.zeros((rows, d.talker.hidden), dtype=torch.int16, device=self.dev)
        self.pf_logits0 = torch.zeros((self.B, d.talker_vocab), dtype=torch.float32, device=self.dev)
        self.pf_tok0 = torch.zeros(self.B, dtype=torch.int32, device=self.dev)
        self.pf_h = torch.zeros((self.B, d.talker.hidden), dtype=torch.int16, device=self.dev)

    def _pf_args(self):
        return PrefillArgs(self.pf_rows, self.B, self.pf_seq_start.data_ptr(),
                           self.pf_embeds.data_ptr(), self.page_table.data_ptr(), self.max_pages,
                           self.kv_len.data_ptr(), self.pf_logits0.data_ptr(),
                           self.pf_tok0.data_ptr(), self.pf_h.data_ptr(), self.status.data_ptr())

    def prefill_inputs(self, prompts):
        """Pack prompts (per session: bf16 bits [T_s, hidden], or None) into the rows."""
        torch = self.torch
        starts = [0]
        rows = np.zeros((self.pf_rows, self.dims.talker.hidden), dtype=np.uint16)
        for b in range(self.B):
            p = prompts[b] if b < len(prompts) and prompts[b] is not None else None
            n = 0 if p is None else p.shape[0]
            if starts[-1] + n > self.pf_rows:
                raise ValueError("prompts exceed the prefill rows")
            if n:
                rows[starts[-1]:starts[-1] + n] = p
            starts.append(starts[-1] + n)
        self.pf_seq_start.copy_(torch.as_tensor(np.asarray(starts, dtype=np.int32)))
        self.pf_embeds.copy_(_bits(torch, rows, self.dev))

    def prefill(self):
        """Enqueue a prefill of the packed prompts on the current stream."""
        qt_prefill(self.model, self._pf_args(), self._kv(), self.pf_ws_ptr, self.pf_ws_bytes,
                   self.torch.cuda.current_stream(self.dev).cuda_stream)

    def prefill_capture(self) -> int:
        g = qt_prefill_graph_create(self.model, self._pf_args(), self._kv(), self.pf_ws_ptr,
                                    self.pf_ws_bytes)
        self.graphs.append(g)
        return g

    def _kv(self):
        return KvCaches(self.k_pages.data_ptr(), self.v_pages.data_ptr(), self.num_pages)

    def trace(self, mode: str = "full", forced: bool = False, sampling: bool = False):
        """Run one frame as decode() does with an event around every launch; waits for
        it and returns [(kernel name, kind, info, ms)] in launch order."""
        if self._trace is None:
            self._trace_n = qt_frame_launch_count(self.cfg, MODES["full"], self.B)
            self._trace = qt_trace_create(self._trace_n)
        ss, kv, fi, fo = self._descs(mode, forced, sampling=sampling)
        qt_frame_trace(self.model, ss, kv, fi, fo, self.ws_ptr, self.ws_bytes,
                       self.torch.cuda.current_stream(self.dev).cuda_stream, self._trace)
        return [(li.name.decode(), KERNEL_KINDS[li.kind], li, ms)
                for li, ms in qt_trace_read(self._trace, self._trace_n)]

    def capture(self, mode: str = "full", forced: bool = False, sampling: bool = False) -> int:
        ss, kv, fi, fo = self._descs(mode, forced, sampling=sampling)
        g = qt_frame_graph_create(self.model, ss, kv, fi, fo, self.ws_ptr, self.ws_bytes)
        self.graphs.append(g)
        return g

    def replay(self, graph: int):
        qt_frame_graph_launch(graph, self.torch.cuda.current_stream(self.dev).cuda_stream)

    def close(self):
        for g in self.graphs:
            qt_graph_destroy(g)
        self.graphs = []
        if self._trace is not None:
            qt_trace_destroy(self._trace)
            self._trace = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def setup_workload(w, model: PackedModel, kv_pool=None):
    """A Decoder for workload `w` (a synth.Workload) with every session's
    prefilled Talker cache laid out into its pages.  Returns (decoder, lengths)."""
    import synth
    from concurrent.futures import ThreadPoolExecutor
    d = w.dims
    lengths = w.lengths()
    dec = Decoder(model, batch=w.batch, max_pages=w.max_pages())
    if w.mode != "predictor":
        t = d.talker
        with ThreadPoolExecutor(synth._threads()) as pool:
            for b in range(w.batch):
                if kv_pool is not None and b in kv_pool:
                    kb, vb = kv_pool[b]
                else:
                    kb, vb = synth.gen_kv(w.name, b, t.layers, int(lengths[b]), t.n_kv, t.head_dim,
                                          pool=pool)
                dec.load_session_kv(b, kb, vb)
    dec.torch.cuda.synchronize(dec.dev)
    return dec, lengths


class Scheduler:
    """The library's lockstep scheduler (qt_sched.h) with its buffers: a Talker KV
    pool of num_pages pages, the scheduler's device buffer and its pinned host
    buffer.  Every step enqueues on the stream current at construction."""

    def __init__(self, model: PackedModel, buckets=(1, 2, 4, 8, 16, 32), max_sessions: int = 32,
                 max_pages: int = 8, num_pages: int | None = None, eos_index: int = -1):
        import torch
        self.torch = torch
        self.pm = model
        self.dims = model.dims
        self.dev = model.dev
        t = self.dims.talker
        self.num_pages = num_pages if num_pages is not None else max_sessions * max_pages + 1
        self.max_pages = max_pages
        self.scfg = make_sched_cfg(buckets, max_sessions, max_pages, eos_index)
        dev_bytes, host_bytes = qt_sched_bytes(model.cfg, self.scfg)
        self._dev_buf, self.dev_ptr = _aligned(torch, dev_bytes, self.dev)
        self._dev_off = self.dev_ptr - self._dev_buf.data_ptr()
        self._host_buf = torch.empty(host_bytes + 256, dtype=torch.uint8, pin_memory=True)
        self.host_ptr = self._host_buf.data_ptr() + (-self._host_buf.data_ptr()) % 256
        shape = (t.layers, self.num_pages, t.n_kv, PAGE, t.head_dim)
        self.k_pages = torch.zeros(shape, dtype=torch.int16, device=self.dev)
        self.v_pages = torch.zeros(shape, dtype=torch.int16, device=self.dev)
        self.kv = KvCaches(self.k_pages.data_ptr(), self.v_pages.data_ptr(), self.num_pages)
        self.stream = torch.cuda.current_stream(self.dev)
        self.handle = qt_sched_create(model.handle, self.scfg, self.kv, self.dev_ptr, dev_bytes,
                                      self.host_ptr, host_bytes, self.stream.cuda_stream)
        self._held = []

    def _view(self, ptr: int, dtype, shape):
        torch = self.torch
        esize = torch.tensor([], dtype=dtype).element_size()
        off = ptr - self._dev_buf.data_ptr()
        n = int(np.prod(shape))
        return self._dev_buf[off:off + n * esize].view(dtype).view(*shape)

    def open(self, length: int, k_bits=None, v_bits=None, min_frames: int = 1,
             max_frames: int = 1 << 30, copy_from=None) -> int:
        """Open a session with `length` prefilled positions, written into the pages the
        scheduler hands out: from K/V bits [layers, length, n_kv, hd], or copied on
        the device from copy_from = (k_pool, v_pool, page ids in position order) of
        another pool with the same layout."""
        sid, pages = qt_sched_open(self.handle, length, min_frames, max_frames, PAGE)
        torch = self.torch
        with torch.cuda.stream(self.stream):  # ordered before the session's first step
            if length and copy_from is not None:
                k_src, v_src, src_pages = copy_from
                dst = torch.as_tensor(np.asarray(pages, dtype=np.int64), device=self.dev)
                src = torch.as_tensor(np.asarray(src_pages[:len(pages)], dtype=np.int64),
                                      device=self.dev)
                self.k_pages[:, dst] = k_src[:, src]
                self.v_pages[:, dst] = v_src[:, src]
            elif length:
                _write_pages(torch, self.k_pages, self.v_pages, pages, k_bits, v_bits)
        return sid

    def open_pages(self, length: int, min_frames: int = 1, max_frames: int = 1 << 30):
        """Open a session with `length` positions to be prefilled and return (id, its
        pages in position order) without writing them: the caller fills them, e.g.
        with prefill() below, before the session's first step."""
        sid, pages = qt_sched_open(self.handle, length, min_frames, max_frames, PAGE)
        return sid, [int(p) for p in pages]

    def prefill(self, sessions, prompts):
        """qt_prefill of prompts[i] (bf16 bits [T_i, talker hidden], T_i the length the
        session was opened with) into the pages of sessions[i] = (id, pages) from
        open_pages, on this scheduler's stream.  Returns device tensors (logits0
        [n, talker_vocab], tok0 [n], h_last bf16 bits [n, talker hidden], status [1]),
        valid once the stream has reached them."""
        torch, d = self.torch, self.dims
        n = len(sessions)
        lens = [int(p.shape[0]) for p in prompts]
        rows = max(16, -(-sum(lens) // 16) * 16)
        if rows > 64:
            rows = -(-rows // 64) * 64
        starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        emb = np.zeros((rows, d.talker.hidden), dtype=np.uint16)
        table = np.zeros((n, self.max_pages), dtype=np.int32)
        for i, ((_, pages), p) in enumerate(zip(sessions, prompts)):
            emb[starts[i]:starts[i + 1]] = p
            table[i, :len(pages)] = pages
            table[i, len(pages):] = pages[-1] if pages else 0  # (past the prompt: never used)
        dev = self.dev
        with torch.cuda.stream(self.stream):  # the copies, the call and its steps share one stream
            bufs = {
                "seq_start": torch.from_numpy(starts).to(dev),
                "embeds": torch.from_numpy(emb.view(np.int16)).to(dev),
                "page_table": torch.from_numpy(table).to(dev),
                "kv_len": torch.zeros(n, dtype=torch.int32, device=dev),
                "logits0": torch.zeros((n, d.talker_vocab), dtype=torch.float32, device=dev),
                "tok0": torch.zeros(n, dtype=torch.int32, device=dev),
                "h_last": torch.zeros((n, d.talker.hidden), dtype=torch.int16, device=dev),
                "status": torch.zeros(1, dtype=torch.int32, device=dev),
            }
            ws_bytes = qt_prefill_workspace_bytes(self.pm.cfg, rows, n)
            ws_buf, ws_ptr = _aligned(torch, ws_bytes, dev)
            args = PrefillArgs(rows, n, bufs["seq_start"].data_ptr(), bufs["embeds"].data_ptr(),
                               bufs["page_table"].data_ptr(), self.max_pages,
                               bufs["kv_len"].data_ptr(), bufs["logits0"].data_ptr(),
                               bufs["tok0"].data_ptr(), bufs["h_last"].data_ptr(),
                               bufs["status"].data_ptr())
            qt_prefill(self.pm.handle, args, self.kv, ws_ptr, ws_bytes, self.stream.cuda_stream)
        self._held.append((bufs, ws_buf))  # alive until the next step is enqueued
        return bufs["logits0"], bufs["tok0"], bufs["h_last"], bufs["status"]

    def set_sampling(self, sid: int, params=None, seed: int = 0):
        """params: (codebook-0, predictor) (temperature, top_p, penalty, top_k) pair, or
        None for greedy."""
        qt_sched_set_sampling(self.handle, sid, params, seed)

    def submit(self, sid: int, talker_in, forced=None):
        """talker_in: device int16 [talker hidden] (bf16 bits); forced: device int32
        [n_codebooks] or None.  The step reads them on the scheduler's stream, so they
        are recorded as in use there: the caching allocator does not hand their memory
        out again until the step that reads them has run, whatever stream the caller
        allocated them on."""
        qt_sched_submit(self.handle, sid, talker_in.data_ptr(),
                        forced.data_ptr() if forced is not None else None)
        talker_in.record_stream(self.stream)
        if forced is not None:
            forced.record_stream(self.stream)
        self._held.append((talker_in, forced))

    def step(self) -> int:
        n = qt_sched_step(self.handle)
        self._held = []
        return n

    def outputs(self, sid: int):
        """(logits0 [talker_vocab], logits_pred [n_codebooks-1, code_vocab], tokens
        [n_codebooks], frames) as views of the scheduler's device buffer."""
        torch, d = self.torch, self.dims
        l0, lp, tok, frames = qt_sched_outputs(self.handle, sid)
        return (self._view(l0, torch.float32, (d.talker_vocab,)),
                self._view(lp, torch.float32, (d.n_steps, d.code_vocab)),
                self._view(tok, torch.int32, (d.n_codebooks,)), frames)

    def state(self, sid: int):
        return qt_sched_state(self.handle, sid)

    def length(self, sid: int) -> int:
        return qt_sched_length(self.handle, sid)

    def free_pages(self) -> int:
        return qt_sched_free_pages(self.handle)

    def close_session(self, sid: int):
        qt_sched_close(self.handle, sid)

    def status(self) -> int:
        return int(self._view(qt_sched_status_word(self.handle), self.torch.int32, (1,)).item())

    def close(self):
        if self.handle:
            qt_sched_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
