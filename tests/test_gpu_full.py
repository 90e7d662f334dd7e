"""Full-size workloads on the GPU, in the launch configuration bench.py times,
compared element by element with the float32 oracle: every element of Y, dX,
the four LoRA gradients (each expert's slice normed by itself) and the
routing-weight and logit gradients, with every reference computed from the
oracle's own routing (top-k ids equal to the GPU's bit for bit, routing
weights the oracle's).  A rerun in the same buffers must reproduce every
output bit for bit.  The headline shape runs again with fp16 elements.
Routing at these sizes is compared in full by test_gpu_route.

Oracle time on 16 host threads (float32 numpy, forward + backward): about 2 s
for qwen3_30b_a3b, 3 s for deepseek_shared and 10-20 s each for long_zipf and
routing_stress."""
import time
from dataclasses import replace

import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel
import oracle
from gpu_helpers import TOL, announce, compare_layer, mdims, require_gpu, upload
from synth import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

FULL = {name: CONFIGS[name] for name in
        ("qwen3_30b_a3b", "deepseek_shared", "long_zipf", "routing_stress")}
FULL["qwen3_30b_a3b_f16"] = replace(CONFIGS["qwen3_30b_a3b"], element="f16")


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_every_element(name):
    require_gpu()
    ld = FULL[name]
    announce("full", name, ld)
    inp = make_inputs(ld, seed=0)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    layer = mel.MoELoRALayer(dims, w)
    layer.y.fill_(float("nan"))
    for t in layer.grads:
        t.fill_(float("nan"))
    layer.route(logits)
    y = layer.forward(x)
    g = layer.backward(dy, x, router=True)
    torch.cuda.synchronize()
    first = [t.clone() for t in (y, g.dx, g.da_gate_up, g.db_gate_up, g.da_down, g.db_down,
                                 layer.router_grads.d_topk_w, layer.router_grads.d_logits)]
    # a second route + forward + backward in the same buffers gives bitwise the
    # same outputs (no atomics, no order that depends on timing)
    layer.route(logits)
    layer.forward(x)
    layer.backward(dy, x, router=True)
    torch.cuda.synchronize()
    again = (layer.y, g.dx, g.da_gate_up, g.db_gate_up, g.da_down, g.db_down,
             layer.router_grads.d_topk_w, layer.router_grads.d_logits)
    for a, b in zip(first, again):
        assert torch.equal(a, b), "a rerun changed an output"

    t0 = time.perf_counter()
    ids, tw = oracle.topk_softmax(inp.logits, ld.k)
    np.testing.assert_array_equal(layer.routing.topk_ids.cpu().numpy(), ids)
    np.testing.assert_allclose(layer.routing.topk_w.cpu().numpy(), tw, rtol=2e-6, atol=1e-7)
    fw = oracle.forward(inp, ids, tw, ld, dtype=np.float32)
    bw = oracle.backward(inp, ids, tw, ld, dtype=np.float32)
    rgr = oracle.router_grads(inp, ids, tw, ld, dtype=np.float32, fw=fw)
    print(f"oracle {time.perf_counter() - t0:.1f} s", flush=True)
    got = {"y": y, "dx": g.dx, "da_gu": g.da_gate_up, "db_gu": g.db_gate_up,
           "da_dn": g.da_down, "db_dn": g.db_down, "d_topk_w": layer.router_grads.d_topk_w,
           "d_logits": layer.router_grads.d_logits}
    errs = compare_layer(got, fw, bw, rgr)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for key, e in errs.items():
        assert e <= TOL, (key, e)
