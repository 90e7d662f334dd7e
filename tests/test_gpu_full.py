"""Full-size workloads on the GPU, in the launch configuration bench.py times,
checked against the oracle on outputs it can compute one by one: Y, dX and
router-gradient rows of sampled tokens (float64), and the LoRA gradients of
sampled experts (float32: the least-loaded expert with rows, an empty expert
when there is one, the most-loaded expert, and the shared expert when there
is one), and a rerun in the same buffers must reproduce every output bit for
bit.  The headline shape runs again with fp16 elements.
Routing at these sizes is compared in full by test_gpu_route."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel
import oracle
from gpu_helpers import TOL, announce, mdims, relerr, require_gpu, to_numpy_f64, upload
from synth import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

FULL = {name: CONFIGS[name] for name in
        ("qwen3_30b_a3b", "deepseek_shared", "long_zipf", "routing_stress")}
FULL["qwen3_30b_a3b_f16"] = replace(CONFIGS["qwen3_30b_a3b"], element="f16")


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled(name):
    require_gpu()
    ld = FULL[name]
    announce("full", name, ld)
    inp = make_inputs(ld, seed=0)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    layer = mel.MoELoRALayer(dims, w)
    for t in layer.grads:
        t.fill_(float("nan"))
    layer.route(logits)
    y = layer.forward(x)
    g = layer.backward(dy, x, router=True)
    torch.cuda.synchronize()
    ids = layer.routing.topk_ids.cpu().numpy()
    tw = layer.routing.topk_w.cpu().numpy()
    np.testing.assert_array_equal(ids, oracle.topk_softmax(inp.logits, ld.k)[0])
    rng = np.random.default_rng(7)
    toks = sorted(set([0, ld.T - 1] + rng.choice(ld.T, 4, replace=False).tolist()))
    y_ref = oracle.forward_tokens(inp, ids, tw, ld, toks)
    dx_ref = oracle.backward_tokens(inp, ids, tw, ld, toks)
    ey = relerr(to_numpy_f64(y)[toks], y_ref)
    edx = relerr(to_numpy_f64(g.dx)[toks], dx_ref)
    r_ref = oracle.router_grads_tokens(inp, ids, tw, ld, toks)
    edw = relerr(to_numpy_f64(layer.router_grads.d_topk_w)[toks], r_ref["d_topk_w"])
    edl = relerr(to_numpy_f64(layer.router_grads.d_logits)[toks], r_ref["d_logits"])
    print(f"Y rows {ey:.2e}  dX rows {edx:.2e}  d_topk_w rows {edw:.2e}  d_logits rows {edl:.2e}",
          flush=True)
    assert ey <= TOL and edx <= TOL and edw <= TOL and edl <= TOL
    counts = np.bincount(ids.reshape(-1), minlength=ld.E)
    experts = {int(np.argmin(np.where(counts > 0, counts, 1 << 30))), int(np.argmax(counts))}
    if np.any(counts == 0):
        experts.add(int(np.argmin(counts)))
    if ld.n_shared:
        experts.add(ld.E)
    got = [to_numpy_f64(t) for t in (g.da_gate_up, g.db_gate_up, g.da_down, g.db_down)]
    for a in got:
        assert np.all(np.isfinite(a)), "unwritten or non-finite gradient elements"
    # a second route + forward + backward in the same buffers gives bitwise the
    # same outputs (no atomics, no order that depends on timing)
    first = [t.clone() for t in (y, g.dx, g.da_gate_up, g.db_gate_up, g.da_down, g.db_down,
                                 layer.router_grads.d_topk_w, layer.router_grads.d_logits)]
    layer.route(logits)
    layer.forward(x)
    layer.backward(dy, x, router=True)
    torch.cuda.synchronize()
    again = (layer.y, g.dx, g.da_gate_up, g.db_gate_up, g.da_down, g.db_down,
             layer.router_grads.d_topk_w, layer.router_grads.d_logits)
    for a, b in zip(first, again):
        assert torch.equal(a, b), "a rerun changed an output"
    for e in sorted(experts):
        ref = oracle.lora_grads_expert(inp, ids, tw, ld, e, dtype=np.float32)
        errs = [relerr(a[e], b) if np.any(b) else float(np.max(np.abs(a[e]))) for a, b in zip(got, ref)]
        print(f"expert {e} rows {counts[e] if e < ld.E else ld.T}: " + " ".join(f"{v:.2e}" for v in errs),
              flush=True)
        for v in errs:
            assert v <= TOL, (e, errs)
