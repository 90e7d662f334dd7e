"""The binding on a stream other than the current one, and the per-thread
kernel-timing recorder.

* route / forward / backward given a side stream (with every temporary
  allocated by the wrappers) give bitwise the results of the same calls on
  the current stream, after the side stream is synchronised;
* one thread's recorder sees only the kernels that thread launched;
* two layers running at once on two streams each give bitwise their results
  alone."""
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


LD_B = LayerDims(1500, 128, 192, 12, 4, 8)


def _step(layer, logits, x, dy, stream):
    layer.route(logits, stream=stream)
    layer.forward(x, stream=stream)
    layer.backward(dy, x, stream=stream, router=True)


def _outs(layer):
    rg = layer.router_grads
    return [*layer.routing, layer.y, *layer.grads, rg.d_topk_w, rg.d_logits]


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_two_layers_on_two_streams_at_once():
    """Two layers of different shapes, each with its own buffers, run their
    steps interleaved on two streams with no wait in between: each must give
    bitwise what it gives alone on the current stream (no device state is
    shared between calls on different streams)."""
    require_gpu()
    announce("two streams", LD, LD_B)
    cases = []
    for ld, seed in ((LD, 8), (LD_B, 9)):
        inp = make_inputs(ld, seed=seed)
        dims = mdims(ld)
        logits, x, dy, w = upload(inp)
        cases.append((mel.MoELoRALayer(dims, w), logits, x, dy))
    ref = []
    for layer, logits, x, dy in cases:
        _step(layer, logits, x, dy, None)
        torch.cuda.synchronize()
        ref.append([t.clone() for t in _outs(layer)])
    for layer, *_ in cases:
        for t in _outs(layer):
            t.fill_(-1 if not t.dtype.is_floating_point else float("nan"))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())  # the refills above
    for _ in range(3):  # several steps each, queued together
        for (layer, logits, x, dy), s in zip(cases, streams):
            _step(layer, logits, x, dy, s)
    torch.cuda.synchronize()
    for (layer, *_), r in zip(cases, ref):
        for i, (a, b) in enumerate(zip(r, _outs(layer))):
            assert torch.equal(_bits(a), _bits(b)), f"output {i} differs"
