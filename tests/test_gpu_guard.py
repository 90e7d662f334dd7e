"""Guard bands: every buffer the library writes (routing outputs, Y, the
saved activations, both workspaces, dX, the LoRA gradients and the router
gradients) sits inside a larger allocation whose 4 KiB before and after are
filled with a byte pattern; after route + forward + backward on each engine,
those bands must be untouched (no write past either end of any buffer), and
the outputs must equal a run in plain allocations bit for bit."""
import pytest
import torch

import mixture_experts_lora_amd as mel
from gpu_helpers import announce, mdims, require_gpu, upload
from synth import LayerDims, make_inputs

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5

CASES = {
    "tiny": LayerDims(256, 128, 64, 8, 2, 4),
    "ragged_shared_r3_s2": LayerDims(333, 192, 128, 6, 2, 3, n_shared=1, lora_scale=2.0),
    "r128_n192": LayerDims(200, 128, 192, 4, 2, 128),
    "empty_experts_r64": LayerDims(300, 128, 64, 28, 6, 64, logits_recipe="stress"),
    "splitk_two_chunks": LayerDims(2500, 128, 64, 2, 2, 16),
    "one_token": LayerDims(1, 64, 64, 4, 2, 4),
    "wide_d320_zipf_f16": LayerDims(700, 320, 192, 8, 3, 24, logits_recipe="zipf", element="f16"),
}


class Arena:
    """Buffers carved out of guarded allocations."""

    def __init__(self):
        self.blocks = []

    def take(self, shape, dtype):
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((GUARD + nbytes + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.blocks.append(raw)
        return raw[GUARD:GUARD + nbytes].view(dtype).view(*shape)

    def intact(self):
        bad = []
        for i, raw in enumerate(self.blocks):
            if not (bool((raw[:GUARD] == PATTERN).all()) and bool((raw[-GUARD:] == PATTERN).all())):
                bad.append(i)
        return bad


def _run_guarded(dims, logits, x, dy, w):
    A = Arena()
    T, k, E, P, Et = dims.T, dims.k, dims.E, dims.P, dims.E_tot
    d, n, r = dims.d, dims.n, dims.r
    i32, f32 = torch.int32, torch.float32
    rt = mel.Routing(A.take((T, k), i32), A.take((T, k), f32), A.take((E,), i32),
                     A.take((E + 1,), i32), A.take((P,), i32), A.take((P,), i32),
                     A.take((dims.P_tot,), i32), A.take((dims.P_tot,), f32))
    rws = A.take((mel.route_workspace_bytes(dims),), torch.uint8)
    saved = A.take((mel.forward_saved_bytes(dims),), torch.uint8)
    ws = A.take((mel.workspace_bytes(dims),), torch.uint8)
    y = A.take((T, d), dims.elem)
    g = mel.Grads(A.take((T, d), dims.elem), A.take((Et, d, r), f32), A.take((Et, r, 2 * n), f32),
                  A.take((Et, n, r), f32), A.take((Et, r, d), f32))
    rg = mel.RouterGrads(A.take((T, k), f32), A.take((T, E), f32))
    mel.route(logits, dims, rt, rws)
    mel.forward(x, rt, w, dims, y, saved, ws)
    mel.backward(dy, x, rt, w, saved, dims, g, ws, router_out=rg)
    torch.cuda.synchronize()
    return A, rt, y, g, rg


def _run_plain(dims, logits, x, dy, w):
    rt = mel.route(logits, dims)
    y, saved = mel.forward(x, rt, w, dims)
    rg = mel.empty_router_grads(dims, "cuda")
    g = mel.backward(dy, x, rt, w, saved, dims, router_out=rg)
    torch.cuda.synchronize()
    return rt, y, g, rg


@pytest.mark.parametrize("engines", [mel.ENGINE_ALL, 0], ids=["streamed", "register_path"])
@pytest.mark.parametrize("name", list(CASES))
def test_no_write_outside_buffers(name, engines):
    require_gpu()
    ld = CASES[name]
    announce("guard", f"{name} engines={engines}", ld)
    inp = make_inputs(ld, seed=3)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    before = mel.get_engines(dims)
    mel.set_engines(dims, engines)
    try:
        A, rt, y, g, rg = _run_guarded(dims, logits, x, dy, w)
        rt2, y2, g2, rg2 = _run_plain(dims, logits, x, dy, w)
    finally:
        mel.set_engines(dims, before)
    assert A.intact() == [], f"guard bands overwritten in buffers {A.intact()}"
    for a, b in zip(list(rt) + [y] + list(g) + list(rg), list(rt2) + [y2] + list(g2) + list(rg2)):
        assert torch.equal(a.view(torch.int16) if a.dtype == dims.elem else a,
                           b.view(torch.int16) if b.dtype == dims.elem else b)
