"""Forward and backward on the GPU against the float64 oracle, element by
element, at sizes the oracle finishes in seconds: several M/N tiles, ragged
segment tails, ranks that are and are not multiples of 8 (rank 1 included), a
shared expert, LoRA scales of 2, 0 and -0.75, empty experts, split-K LoRA
gradients, k = E, k = 1, T = 1, a single expert, the largest expert count (256
with the shared one); the routing-weight and logit gradients with every case;
every case again with fp16 elements.

Every reference is the oracle's, from the oracle's own routing (its top-k ids,
which the GPU's must equal bit for bit, and its routing weights, which the
GPU's must equal to fp32 rounding).  Y, dX and the router gradients are
normed over the whole tensor, each expert's LoRA gradients over that expert's
slice.  Every output buffer is filled with NaN before the call (an unwritten
element fails), and the whole route + forward + backward runs twice with
bitwise equal results (no races, no order-dependent sums)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel
import oracle
from gpu_helpers import TOL, announce, compare_layer, mdims, require_gpu, to_numpy_f64, upload
from synth import CONFIGS, LayerDims, make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": CONFIGS["tiny"],
    "ragged_shared_r3_s2": LayerDims(333, 192, 128, 6, 2, 3, n_shared=1, lora_scale=2.0),
    "r128_n192": LayerDims(200, 128, 192, 4, 2, 128),
    "empty_experts_r64": LayerDims(300, 128, 64, 28, 6, 64, logits_recipe="stress"),
    "splitk_two_chunks": LayerDims(2500, 128, 64, 2, 2, 16),
    "k_equals_E": LayerDims(64, 64, 64, 4, 4, 8),
    "k_one": LayerDims(96, 64, 64, 4, 1, 8),
    "one_token": LayerDims(1, 64, 64, 4, 2, 4),
    "wide_d320_zipf": LayerDims(700, 320, 192, 8, 3, 24, logits_recipe="zipf"),
    # contraction long enough for the rank-r pre-passes to split over workgroups
    "prepass_splits": LayerDims(200, 1024, 256, 4, 2, 16),
    # the most experts the library takes: 255 routed + 1 shared = 256, most of them empty or tiny
    "max_experts_255_shared": LayerDims(600, 64, 64, 255, 4, 8, n_shared=1),
    # rank 1: one column of each adapter
    "rank_one": LayerDims(150, 64, 128, 4, 2, 1),
    # one expert, k = 1: every token's weight is 1, the layer is one dense SwiGLU MLP with LoRA
    "single_expert": LayerDims(130, 128, 64, 1, 1, 8),
    # LoRA scale 0: only the base path is left and every LoRA gradient is exactly zero
    "scale_zero": LayerDims(100, 64, 64, 4, 2, 8, lora_scale=0.0),
    "scale_negative_shared": LayerDims(90, 64, 64, 3, 2, 5, n_shared=1, lora_scale=-0.75),
}
CASES.update({f"{k}_f16": replace(v, element="f16") for k, v in list(CASES.items())})


def _run(dims, logits, x, dy, w):
    rt = mel.route(logits, dims)
    y = torch.full((dims.T, dims.d), float("nan"), dtype=dims.elem, device="cuda")
    y, saved = mel.forward(x, rt, w, dims, y=y)
    g = mel.empty_grads(dims, "cuda")
    rg = mel.empty_router_grads(dims, "cuda")
    for t in list(g) + list(rg):
        t.fill_(float("nan"))
    g = mel.backward(dy, x, rt, w, saved, dims, out=g, router_out=rg)
    torch.cuda.synchronize()
    return rt, y, g, rg


@pytest.mark.parametrize("name", list(CASES))
def test_layer_parity(name):
    require_gpu()
    ld = CASES[name]
    announce("layer", name, ld)
    inp = make_inputs(ld, seed=1)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    rt, y, g, rg = _run(dims, logits, x, dy, w)
    ids, tw = oracle.topk_softmax(inp.logits, ld.k)
    np.testing.assert_array_equal(rt.topk_ids.cpu().numpy(), ids)
    np.testing.assert_allclose(rt.topk_w.cpu().numpy(), tw, rtol=2e-6, atol=1e-7)
    fw = oracle.forward(inp, ids, tw, ld)
    bw = oracle.backward(inp, ids, tw, ld)
    rgr = oracle.router_grads(inp, ids, tw, ld, fw=fw)
    got = {"y": y, "dx": g.dx, "da_gu": g.da_gate_up, "db_gu": g.db_gate_up,
           "da_dn": g.da_down, "db_dn": g.db_down, "d_topk_w": rg.d_topk_w,
           "d_logits": rg.d_logits}
    errs = compare_layer(got, fw, bw, rgr)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for key, e in errs.items():
        assert e <= TOL, (key, e)
    # experts without rows get exactly zero LoRA gradients
    counts = np.bincount(ids.reshape(-1), minlength=ld.E)
    for e in np.nonzero(counts == 0)[0]:
        for key in ("da_gu", "db_gu", "da_dn", "db_dn"):
            assert not np.any(to_numpy_f64(got[key])[e]), (key, e)
    # with LoRA scale 0 every adapter gradient is a sum of products with a zero factor
    if ld.lora_scale == 0:
        for key in ("da_gu", "db_gu", "da_dn", "db_dn"):
            assert not np.any(to_numpy_f64(got[key])), key
    # bitwise reproducible
    rt2, y2, g2, rg2 = _run(dims, logits, x, dy, w)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    for a, b in zip(list(g) + list(rg), list(g2) + list(rg2)):
        assert torch.equal(a.view(torch.int16) if a.dtype == dims.elem else a,
                           b.view(torch.int16) if b.dtype == dims.elem else b)


ENGINE_CASES = ["tiny", "ragged_shared_r3_s2", "r128_n192", "empty_experts_r64", "splitk_two_chunks",
                "wide_d320_zipf", "ragged_shared_r3_s2_f16", "empty_experts_r64_f16",
                "wide_d320_zipf_f16"]


ALL4 = sum(1 << p for p in range(4))
SETTINGS = {
    "register_path": 0,
    "streamed": mel.ENGINE_ALL,
    "streamed_256rows": mel.ENGINE_ALL | (ALL4 << 5),
    "streamed_32k": mel.ENGINE_ALL | (ALL4 << 9),
    "streamed_256rows_32k": mel.ENGINE_ALL | (ALL4 << 5) | (ALL4 << 9),
    "splitk_1024": mel.ENGINE_ALL | mel.SPLITK_1024,
    "splitk_4096": mel.ENGINE_ALL | mel.SPLITK_4096,
    "mixed": (mel.ENGINE_ALL & ~mel.ENGINE_DOWN) | mel.TILE256(0) | mel.STAGE32(2) | mel.TILE256(3)
             | mel.STAGE32(3) | mel.SPLITK_1024,
}


@pytest.mark.parametrize("engines", list(SETTINGS.values()), ids=list(SETTINGS))
@pytest.mark.parametrize("name", ENGINE_CASES)
def test_layer_parity_each_engine(name, engines):
    """Every product under one setting the autotune can choose: all
    register-path kernels, all streamed in each tile configuration (320 or
    256 rows, 64- or 32-k stages), each split-K chunk of the LoRA gradients,
    and one mixed setting."""
    require_gpu()
    ld = CASES[name]
    announce("engines", f"{name} engines={engines}", ld)
    inp = make_inputs(ld, seed=2)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    before = mel.get_engines(dims)
    mel.set_engines(dims, engines)
    try:
        assert mel.get_engines(dims) == engines
        rt, y, g, rg = _run(dims, logits, x, dy, w)
    finally:
        mel.set_engines(dims, before)
    ids, tw = oracle.topk_softmax(inp.logits, ld.k)
    np.testing.assert_array_equal(rt.topk_ids.cpu().numpy(), ids)
    fw = oracle.forward(inp, ids, tw, ld)
    bw = oracle.backward(inp, ids, tw, ld)
    rgr = oracle.router_grads(inp, ids, tw, ld, fw=fw)
    got = {"y": y, "dx": g.dx, "da_gu": g.da_gate_up, "db_gu": g.db_gate_up,
           "da_dn": g.da_down, "db_dn": g.db_down, "d_topk_w": rg.d_topk_w,
           "d_logits": rg.d_logits}
    errs = compare_layer(got, fw, bw, rgr)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert max(errs.values()) <= TOL, errs


def test_autotune_records_a_choice_that_keeps_parity():
    require_gpu()
    ld = LayerDims(2048, 256, 128, 16, 4, 16)
    announce("autotune", "T2048_d256_n128_E16_k4_r16", ld)
    inp = make_inputs(ld, seed=4)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    before = mel.get_engines(dims)
    try:
        chosen = mel.autotune(dims, logits, x, dy, w)
        print("chosen engines", chosen, flush=True)
        print(mel.describe_engines(chosen), flush=True)
        assert chosen & ~0x7FFF == 0 and (chosen >> 13) & 3 != 3  # a valid engine/tile word
        assert mel.get_engines(dims) == chosen
        rt, y, g, rg = _run(dims, logits, x, dy, w)
    finally:
        mel.set_engines(dims, before)
    ids, tw = oracle.topk_softmax(inp.logits, ld.k)
    np.testing.assert_array_equal(rt.topk_ids.cpu().numpy(), ids)
    fw = oracle.forward(inp, ids, tw, ld)
    bw = oracle.backward(inp, ids, tw, ld)
    got = {"y": y, "dx": g.dx, "da_gu": g.da_gate_up, "db_gu": g.db_gate_up,
           "da_dn": g.da_down, "db_dn": g.db_down}
    errs = compare_layer(got, fw, bw, None)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert max(errs.values()) <= TOL, errs
