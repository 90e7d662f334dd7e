"""A whole layer step (route + forward + backward with the router gradients)
captured as one HIP graph with torch.cuda.graph and replayed.  The library's
launch path allocates nothing, records no memset and never waits on the host,
so the captured step is the eager step.  The test replays it three times;
before each replay the program's own eager work refills every output with
NaN (or -1 for the integer routing tables).  Every replay must then
reproduce the eager outputs bit for bit; the path has no atomics and no
timing-dependent order.  Two layers are used: a small one with a shared
expert and a rank that needs its adapters packed, and the 4096-token
Qwen3-30B-A3B-shaped layer on the streamed kernels."""
import pytest
import torch

import mixture_experts_lora_amd as mel
from gpu_helpers import announce, mdims, require_gpu, upload
from synth import CONFIGS, LayerDims, make_inputs

pytestmark = pytest.mark.gpu

LAYERS = {
    "small_shared_r5": LayerDims(700, 192, 128, 12, 3, 5, n_shared=1, lora_scale=1.5),
    "qwen3_30b_a3b": CONFIGS["qwen3_30b_a3b"],
}


def _outputs(layer):
    g, rg = layer.grads, layer.router_grads
    return [layer.y, *g, rg.d_topk_w, rg.d_logits, *layer.routing]


def _poison(ts):
    for t in ts:
        t.fill_(-1 if not t.dtype.is_floating_point else float("nan"))


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("name", list(LAYERS))
def test_step_replays_as_a_graph(name):
    require_gpu()
    ld = LAYERS[name]
    announce("graph", name, ld)
    inp = make_inputs(ld, seed=4)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    layer = mel.MoELoRALayer(dims, w)

    def step():
        layer.route(logits)
        layer.forward(x)
        layer.backward(dy, x, router=True)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in _outputs(layer)]

    # warm-up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        _poison(_outputs(layer))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, _outputs(layer))):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: output {i} differs from the eager step"
    print(f"{name}: 3 replays bitwise equal to the eager step", flush=True)
