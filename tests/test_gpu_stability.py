"""Many steps in a row on the full-size headline layer (T 4096, d 2048, n 768,
E 128, top-8, r 64): 200 route + forward + backward steps, queued back to
back, each tenth one's outputs compared bit for bit with the first step's.
The pipelined kernels rely on exact memory-counter waits and barriers; a
race among them would show as an occasional bitwise difference.  Run with
the build's default engines and with 32-k stages and 256-row tiles."""
import pytest
import torch

import mixture_experts_lora_amd as mel
from gpu_helpers import announce, mdims, require_gpu, upload
from synth import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

ALL4 = sum(1 << p for p in range(4))
ENGINES = {"default": mel.ENGINE_ALL, "256rows_32k": mel.ENGINE_ALL | (ALL4 << 5) | (ALL4 << 9)}


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("engines", list(ENGINES.values()), ids=list(ENGINES))
def test_200_steps_bitwise_stable(engines):
    require_gpu()
    ld = CONFIGS["qwen3_30b_a3b"]
    announce("stability", f"engines={engines}", ld)
    inp = make_inputs(ld, seed=0)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    before = mel.get_engines(dims)
    mel.set_engines(dims, engines)
    try:
        layer = mel.MoELoRALayer(dims, w)

        def step():
            layer.route(logits)
            layer.forward(x)
            layer.backward(dy, x, router=True)

        def outs():
            rg = layer.router_grads
            return [layer.y, *layer.grads, rg.d_topk_w, rg.d_logits, *layer.routing]

        step()
        torch.cuda.synchronize()
        first = [t.clone() for t in outs()]
        snaps = []
        for i in range(1, 200):
            step()
            if i % 10 == 0:
                snaps.append([t.clone() for t in outs()])  # queued, compared at the end
        torch.cuda.synchronize()
    finally:
        mel.set_engines(dims, before)
    for j, snap in enumerate(snaps):
        for k, (a, b) in enumerate(zip(first, snap)):
            assert torch.equal(_bits(a), _bits(b)), f"step {10 * (j + 1)}: output {k} differs"
