"""The autograd wrapper (moe_lora): a loss built on Y back-propagates into x,
the logits and fp32 master copies of the LoRA factors, giving bitwise the
dX, the logit gradient and the (16-bit rounded) factor gradients of the
direct route / forward / backward calls; base weights that require grad are
refused."""
import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel
from gpu_helpers import announce, mdims, require_gpu, upload
from synth import LayerDims, make_inputs

pytestmark = pytest.mark.gpu

LAYERS = {
    "shared_r5": LayerDims(300, 128, 192, 9, 3, 5, n_shared=1, lora_scale=2.0),
    "f16_r16": LayerDims(200, 192, 128, 6, 2, 16, element="f16"),
}


@pytest.mark.parametrize("name", list(LAYERS))
def test_autograd_matches_direct_calls(name):
    require_gpu()
    ld = LAYERS[name]
    announce("autograd", name, ld)
    inp = make_inputs(ld, seed=11)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)

    # direct calls
    rt = mel.route(logits, dims)
    y_ref, saved = mel.forward(x, rt, w, dims)
    rg = mel.empty_router_grads(dims, "cuda")
    g_ref = mel.backward(dy, x, rt, w, saved, dims, router_out=rg)

    # autograd: fp32 master factors, cast to the element type for the layer
    masters = [t.float().requires_grad_() for t in w[2:]]
    xg = x.clone().requires_grad_()
    lg = logits.clone().requires_grad_()
    wl = mel.Weights(w.w_gate_up, w.w_down, *[m.to(dims.elem) for m in masters])
    y = mel.moe_lora(xg, lg, wl, dims)
    (y.float() * dy.float()).sum().backward()
    torch.cuda.synchronize()

    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    assert torch.equal(xg.grad.view(torch.int16), g_ref.dx.view(torch.int16))
    assert torch.equal(lg.grad, rg.d_logits)
    for m, ref in zip(masters, (g_ref.da_gate_up, g_ref.db_gate_up, g_ref.da_down, g_ref.db_down)):
        assert torch.equal(m.grad, ref.to(dims.elem).float())


def test_autograd_refuses_trainable_base_weights():
    require_gpu()
    ld = LAYERS["shared_r5"]
    inp = make_inputs(ld, seed=12)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    w_bad = mel.Weights(w.w_gate_up.clone().requires_grad_(), *w[1:])
    with pytest.raises(ValueError, match="frozen"):
        mel.moe_lora(x, logits, w_bad, dims)
