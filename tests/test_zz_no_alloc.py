"""qt_frame_decode_noalloc (the frame on the library's static scratch) against
qt_frame_decode with a caller workspace: the same kernels, so every output must
agree bit for bit.  Two allocation-free calls run back to back, the second with a
smaller batch, so stale scratch contents from the first cannot leak into it.  A
batch whose workspace exceeds the static scratch is refused before anything is
enqueued."""
import dataclasses

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _frame(dec, L0, noalloc):
    torch = dec.torch
    dec.set_lengths(L0)
    dec.status.zero_()
    dec.logits0.fill_(float("nan"))
    dec.logits_pred.fill_(float("nan"))
    dec.tokens.fill_(-7)
    if noalloc:
        dec.decode_noalloc("full")
    else:
        dec.decode("full")
    torch.cuda.synchronize()
    return {k: getattr(dec, k).cpu().numpy().copy()
            for k in ("logits0", "logits_pred", "tokens", "kv_len", "status")}


def _setup(pm, name, batch, lens, frames=4):
    from streaming_tts_decode_amd.runtime import setup_workload
    w = synth.Workload(name, "full", batch=batch, frames=frames, dims=pm.dims, lens=tuple(lens))
    dec, lengths = setup_workload(w, pm)
    dec.set_inputs(talker_in=synth.frame_inputs(w)["talker_in"][0])
    return dec, lengths


def _check_pair(big, small):
    """big, small: (decoder, lengths).  Reference frames with workspaces first,
    then the two allocation-free calls in a row."""
    ref = [_frame(d, L, noalloc=False) for d, L in (big, small)]
    got = [_frame(d, L, noalloc=True) for d, L in (big, small)]
    for (d, L), r, g in zip((big, small), ref, got):
        assert int(r["status"][0]) == 0
        for k in r:
            np.testing.assert_array_equal(g[k], r[k], err_msg=f"B={d.B}: {k}")
        np.testing.assert_array_equal(g["kv_len"], L + 1)


def test_noalloc_small_model(small_pm):
    big = _setup(small_pm, "noalloc.a", 8, (0, 5, 16, 31, 32, 47, 200, 311))
    small = _setup(small_pm, "noalloc.b", 3, (1, 64, 129))
    _check_pair(big, small)
    for d, _ in (big, small):
        d.close()


def test_noalloc_full_model_b32(full_pm):
    w = synth.WORKLOADS["C4"]
    big = _setup(full_pm, "noalloc.c4", w.batch, w.lengths().tolist(), frames=w.frames)
    small = _setup(full_pm, "noalloc.c3", 6, synth.WORKLOADS["C3"].lengths().tolist())
    _check_pair(big, small)
    for d, _ in (big, small):
        d.close()


def test_noalloc_refuses_oversize(full_pm):
    import streaming_tts_decode_amd as qt
    from streaming_tts_decode_amd import (FrameInputs, FrameOutputs, KvCaches, MODES, QtError,
                                          Sessions)
    torch = full_pm.torch
    cfg = full_pm.cfg
    # a batch whose workspace is larger than the static scratch: refused on the host,
    # before anything is enqueued (the descriptors' buffers are never touched)
    mp = 512
    assert qt.qt_workspace_bytes(cfg, 32, mp) > qt.NOALLOC_SCRATCH_BYTES
    buf = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    p = buf.data_ptr()
    ss = Sessions(32, p, p, mp)
    kv = KvCaches(p, p, 1)
    fi = FrameInputs(MODES["full"], p, p, p, None)
    fo = FrameOutputs(p, p, p, p)
    with pytest.raises(QtError) as e:
        qt.qt_frame_decode_noalloc(full_pm.handle, ss, kv, fi, fo, 0)
    assert e.value.status == 6  # QT_E_CAPACITY
    torch.cuda.synchronize()
    assert int(buf.abs().sum().item()) == 0
