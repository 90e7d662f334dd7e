"""The binding on a stream other than the current one, and the per-thread
kernel-timing recorder.

* route / forward / backward given a side stream (with every temporary
  allocated by the wrappers) give bitwise the results of the same calls on
  the current stream, after the side stream is synchronised;
* one thread's recorder sees only the kernels that thread launched."""
import threading

import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel
from mixture_experts_lora_amd import _lib
from gpu_helpers import announce, mdims, require_gpu, upload
from synth import LayerDims, make_inputs

pytestmark = pytest.mark.gpu

LD = LayerDims(700, 256, 128, 8, 3, 16, n_shared=1)


def _run(dims, logits, x, dy, w, stream):
    rt = mel.route(logits, dims, stream=stream)
    y, saved = mel.forward(x, rt, w, dims, stream=stream)
    g = mel.backward(dy, x, rt, w, saved, dims, stream=stream)
    return rt, y, g


def test_side_stream_matches_current_stream():
    require_gpu()
    announce("side stream", LD)
    inp = make_inputs(LD, seed=6)
    dims = mdims(LD)
    logits, x, dy, w = upload(inp)
    rt0, y0, g0 = _run(dims, logits, x, dy, w, None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    # inputs are produced on the current stream right before the calls: the
    # wrappers must order the side stream after it
    x2 = x * 1
    rt1, y1, g1 = _run(dims, logits, x2, dy, w, side)
    side.synchronize()
    for a, b in zip(list(rt0) + [y0] + list(g0), list(rt1) + [y1] + list(g1)):
        assert torch.equal(a.view(torch.int16) if a.dtype == dims.elem else a,
                           b.view(torch.int16) if b.dtype == dims.elem else b)


def test_timing_recorder_is_per_thread():
    require_gpu()
    announce("per-thread timing", LD)
    inp = make_inputs(LD, seed=7)
    dims = mdims(LD)
    logits, x, dy, w = upload(inp)
    rt = mel.route(logits, dims)
    y, saved = mel.forward(x, rt, w, dims)
    torch.cuda.synchronize()
    go = threading.Event()
    stop = threading.Event()
    errors = []

    def other():
        # forward only, repeatedly, on its own stream, recorder off
        try:
            s = torch.cuda.Stream()
            go.set()
            while not stop.is_set():
                mel.forward(x, rt, w, dims, stream=s)
                s.synchronize()
        except Exception as exc:  # pragma: no cover - reported below
            errors.append(exc)
            go.set()

    th = threading.Thread(target=other)
    th.start()
    go.wait()
    _lib.timing_enable(True)
    for _ in range(3):
        mel.route(logits, dims, out=rt)
    torch.cuda.synchronize()
    rep = _lib.timing_report()
    _lib.timing_enable(False)
    stop.set()
    th.join()
    assert not errors, errors
    # this thread launched only routing: three launches of each routing kernel
    assert set(rep) == {"route_select", "route_scatter"}, rep
    assert all(n == 3 for _, n in rep.values()), rep
