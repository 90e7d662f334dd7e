"""moe_route_noalloc (routing with the library's own per-GPU scratch, for
callers that cannot allocate) against moe_route with a caller workspace,
called through the C ABI: every routing output bit for bit, on two calls in a
row (the second smaller, so it runs over what the first left in the scratch),
recorded into a HIP graph and replayed, and the host-side rejection of a
shape whose scratch would exceed the limit."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel
from mixture_experts_lora_amd import _lib
from gpu_helpers import announce, mdims, require_gpu
from synth import LayerDims, make_logits

pytestmark = pytest.mark.gpu


def _c(dims_l):
    d = mdims(dims_l)
    return d, d.c()


def _filled_routing(dims):
    rt = mel.empty_routing(dims, "cuda")
    for t in rt:  # sentinels: every element must be written
        t.fill_(-7)
    return rt


def _noalloc(lib, dims, dc, logits):
    rt = _filled_routing(dims)
    rc = _lib.MoeRouting(*[t.data_ptr() for t in rt])
    st = lib.moe_route_noalloc(ctypes.byref(dc), logits.data_ptr(), ctypes.byref(rc),
                               torch.cuda.current_stream().cuda_stream)
    assert st == _lib.MOE_SUCCESS, _lib.status_string(st)
    return rt


def _with_workspace(lib, dims, dc, logits):
    rt = _filled_routing(dims)
    rc = _lib.MoeRouting(*[t.data_ptr() for t in rt])
    need = lib.moe_route_workspace_bytes(ctypes.byref(dc))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = lib.moe_route(ctypes.byref(dc), logits.data_ptr(), ctypes.byref(rc), ws.data_ptr(), need,
                       torch.cuda.current_stream().cuda_stream)
    assert st == _lib.MOE_SUCCESS, _lib.status_string(st)
    return rt


def test_noalloc_route_under_graph_capture():
    """The callers it is for: moe_route_noalloc recorded into a HIP graph (in
    a fresh process this is its first call, so its scratch lookup also runs
    during the capture) and replayed three times, the outputs refilled with
    sentinels before each replay; every replay bit for bit equal to moe_route
    with a workspace."""
    require_gpu()
    lib = _lib.load()
    ld = LayerDims(4096, 64, 64, 128, 8, 4)
    announce("route_noalloc graph", ld)
    dims, dc = _c(ld)
    logits = torch.from_numpy(make_logits(ld, seed=30)).cuda()
    ref = _with_workspace(lib, dims, dc, logits)
    rt = _filled_routing(dims)
    rc = _lib.MoeRouting(*[t.data_ptr() for t in rt])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    status = []
    with torch.cuda.graph(graph):
        status.append(lib.moe_route_noalloc(ctypes.byref(dc), logits.data_ptr(), ctypes.byref(rc),
                                            torch.cuda.current_stream().cuda_stream))
    assert status == [_lib.MOE_SUCCESS], _lib.status_string(status[0])
    for rep in range(3):
        for t in rt:
            t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(mel.Routing._fields, rt, ref):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (rep, name)


CALLS = [
    LayerDims(32768, 64, 64, 128, 8, 4, logits_recipe="stress"),  # routing-stress shape, 262,144 pairs
    LayerDims(333, 64, 64, 37, 5, 4, n_shared=1),                 # then a smaller one with a shared expert
]


def test_noalloc_route_matches_workspace_route_twice():
    require_gpu()
    lib = _lib.load()
    for i, ld in enumerate(CALLS):
        announce("route_noalloc", i, ld)
        dims, dc = _c(ld)
        assert lib.moe_route_workspace_bytes(ctypes.byref(dc)) <= _lib.MOE_ROUTE_NOALLOC_SCRATCH_BYTES
        L = make_logits(ld, seed=20 + i)
        L[::97, 3] = np.nan  # non-finite logits take the same path
        logits = torch.from_numpy(L).cuda()
        a = _noalloc(lib, dims, dc, logits)
        b = _with_workspace(lib, dims, dc, logits)
        torch.cuda.synchronize()
        for name, x, y in zip(mel.Routing._fields, a, b):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), name


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    require_gpu()
    lib = _lib.load()
    ld = LayerDims(1 << 20, 64, 64, 8, 1, 4)  # 1 Mi pairs: 4 MiB of ranks alone
    dims, dc = _c(ld)
    assert lib.moe_route_workspace_bytes(ctypes.byref(dc)) > _lib.MOE_ROUTE_NOALLOC_SCRATCH_BYTES
    fake = 4096  # never dereferenced: the size check comes first
    rc = _lib.MoeRouting(*([fake] * 8))
    assert lib.moe_route_noalloc(ctypes.byref(dc), fake, ctypes.byref(rc), None) == \
        _lib.MOE_ERROR_UNSUPPORTED
