"""The largest layers the library accepts, on the GPU.  The kernels address
their per-row buffers with 32-bit byte offsets, so the host checks refuse any
layer whose widest [P_tot, max(2n, d)] buffer reaches 2 GiB (test_abi).  Two
layers sit 64 KiB under that limit (P_tot = 32767 x 8 rows):

  * o_rows   d = 4096: the per-pair outputs O and dX_pair are the large
             buffers;
  * g_rows   2n = 4096: the gate/up rows G and dG are, and H is 1 GiB.

Each runs route + forward + backward with the default streamed kernels and
with the register-path kernels.  Every workspace and saved byte is first set
to 0xFF (a bf16 NaN), so a row that a kernel fails to write reaches Y or dX as
a NaN: every element of Y, dX and both router gradients must come out
finite.  The oracle cannot finish these layers in full within a test, so
values are compared, in float32, where an offset mistake would land:

  * Y, dX and the router gradients of the last tokens routed to the last
    expert (their pairs are the last rows of every per-row buffer), of the
    first tokens routed to expert 0, of the last token and of a seeded sample;
  * the four LoRA gradients of expert 0 and of the last expert (the first
    and the last row segment), each from all of that expert's rows;
  * every token's top-k ids, bit for bit.

Host time per layer: 3-11 s to draw the inputs, 1-5 s of oracle work."""
import time

import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel
import oracle
from gpu_helpers import TOL, announce, mdims, relerr, require_gpu, to_numpy_f64, upload
from synth import LayerDims, make_inputs

pytestmark = pytest.mark.gpu

LAYERS = {
    "o_rows": LayerDims(32767, 4096, 256, 64, 8, 16, lora_scale=0.5, name="o_rows"),
    "g_rows": LayerDims(32767, 256, 2048, 64, 8, 16, lora_scale=0.5, name="g_rows"),
}
ENGINES = {"streamed": mel.ENGINE_ALL, "register_path": 0}
_LIM = 1 << 31


def _sample_tokens(ids: np.ndarray, E: int, T: int) -> np.ndarray:
    last = np.nonzero((ids == E - 1).any(axis=1))[0][-4:]
    first = np.nonzero((ids == 0).any(axis=1))[0][:4]
    rnd = np.random.default_rng(7).choice(T, 8, replace=False)
    return np.unique(np.concatenate([last, first, rnd, [T - 1]]))


@pytest.fixture(scope="module", params=list(LAYERS))
def layer_case(request):
    require_gpu()
    ld = LAYERS[request.param]
    widest = ld.P_tot * max(2 * ld.n, ld.d) * 2
    assert _LIM - (64 << 10) <= widest < _LIM  # just inside the limit
    announce("envelope inputs", request.param, ld)
    inp = make_inputs(ld, seed=3)
    t0 = time.perf_counter()
    ids, tw = oracle.topk_softmax(inp.logits, ld.k)
    toks = _sample_tokens(ids, ld.E, ld.T)
    f32 = np.float32
    ref = {
        "y": oracle.forward_tokens(inp, ids, tw, ld, toks, dtype=f32),
        "dx": oracle.backward_tokens(inp, ids, tw, ld, toks, dtype=f32),
    }
    ref.update({k: v for k, v in
                oracle.router_grads_tokens(inp, ids, tw, ld, toks, dtype=f32).items()})
    experts = (0, ld.E - 1)
    ref["lora"] = {e: oracle.lora_grads_expert(inp, ids, tw, ld, e, dtype=f32) for e in experts}
    print(f"oracle {time.perf_counter() - t0:.1f} s, tokens {toks.tolist()}", flush=True)
    return request.param, ld, inp, ids, toks, experts, ref


@pytest.mark.parametrize("engines", list(ENGINES.values()), ids=list(ENGINES))
def test_envelope_layer(layer_case, engines):
    name, ld, inp, ids, toks, experts, ref = layer_case
    announce("envelope", f"{name} engines={engines}", ld)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    before = mel.get_engines(dims)
    mel.set_engines(dims, engines)
    try:
        layer = mel.MoELoRALayer(dims, w)
        layer.ws.fill_(0xFF)
        layer.saved.fill_(0xFF)
        layer.y.fill_(float("nan"))
        for t in layer.grads:
            t.fill_(float("nan"))
        layer.route(logits)
        y = layer.forward(x)
        g = layer.backward(dy, x, router=True)
        torch.cuda.synchronize()
    finally:
        mel.set_engines(dims, before)
    np.testing.assert_array_equal(layer.routing.topk_ids.cpu().numpy(), ids)
    rg = layer.router_grads
    for key, t in (("y", y), ("dx", g.dx), ("d_topk_w", rg.d_topk_w), ("d_logits", rg.d_logits)):
        assert bool(torch.isfinite(t).all()), f"{key}: unwritten or non-finite elements"
    idx = torch.from_numpy(toks).cuda()
    got = {"y": y[idx], "dx": g.dx[idx], "d_topk_w": rg.d_topk_w[idx], "d_logits": rg.d_logits[idx]}
    errs = {key: relerr(to_numpy_f64(got[key]), ref[key]) for key in got}
    names = ("da_gu", "db_gu", "da_dn", "db_dn")
    mine = (g.da_gate_up, g.db_gate_up, g.da_down, g.db_down)
    for e in experts:
        for key, t, r in zip(names, mine, ref["lora"][e]):
            a = to_numpy_f64(t[e])
            assert np.all(np.isfinite(a)), f"{key}[{e}]: unwritten or non-finite elements"
            errs[f"{key}[{e}]"] = relerr(a, r)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for key, e in errs.items():
        assert e <= TOL, (key, e)
