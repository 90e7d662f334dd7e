"""The merged-weight path the pages compare split LoRA against, on the GPU:
moe_merge_lora's W + s (A B)^T against the oracle's merged weights (every
element within one rounding of the element type, plus the fp32 sum), and
moe_forward_merged's Y against the oracle's merged forward (and the GPU's
split forward against the oracle's split forward on the same inputs), each
element by element at the layer tolerance."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel
import oracle
from gpu_helpers import TOL, announce, mdims, relerr, require_gpu, to_numpy_f64, upload
from synth import CONFIGS, LayerDims, make_inputs

pytestmark = pytest.mark.gpu

UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}

CASES = {
    "tiny": CONFIGS["tiny"],
    "ragged_shared_r3_s2": LayerDims(333, 192, 128, 6, 2, 3, n_shared=1, lora_scale=2.0),
    "r128_n192": LayerDims(200, 128, 192, 4, 2, 128),
    "empty_experts_r64": LayerDims(300, 128, 64, 28, 6, 64, logits_recipe="stress"),
    "wide_d320_zipf": LayerDims(700, 320, 192, 8, 3, 24, logits_recipe="zipf"),
}
CASES.update({f"{k}_f16": replace(v, element="f16") for k, v in list(CASES.items())[:3]})


@pytest.mark.parametrize("name", list(CASES))
def test_merged_weights_and_forward(name):
    require_gpu()
    ld = CASES[name]
    announce("merged", name, ld)
    inp = make_inputs(ld, seed=5)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    rt = mel.route(logits, dims)
    m = mel.MergedWeights(torch.full_like(w.w_gate_up, float("nan")), torch.full_like(w.w_down, float("nan")))
    mel.merge_lora(w, dims, out=m)
    y_m = mel.forward_merged(x, rt, m, dims, y=torch.full_like(x, float("nan")))
    y_s, _ = mel.forward(x, rt, w, dims)
    torch.cuda.synchronize()

    u = UNIT_ROUNDOFF[ld.element]
    for got, ref, nm in zip(m, oracle.merged_weights(inp, ld), ("w_gate_up", "w_down")):
        a = to_numpy_f64(got)
        bound = u * np.abs(ref) + 1e-6 * np.max(np.abs(ref))
        bad = np.abs(a - ref) > bound
        assert not np.any(bad), (nm, int(bad.sum()), float(np.max(np.abs(a - ref))))

    ids, tw = oracle.topk_softmax(inp.logits, ld.k)
    np.testing.assert_array_equal(rt.topk_ids.cpu().numpy(), ids)
    ym_ref = oracle.forward_merged(inp, ids, tw, ld)
    ys_ref = oracle.forward(inp, ids, tw, ld)["y"]
    em = relerr(to_numpy_f64(y_m), ym_ref)
    es = relerr(to_numpy_f64(y_s), ys_ref)
    print(f"merged Y {em:.2e}  split Y {es:.2e}", flush=True)
    assert em <= TOL and es <= TOL


ALL4 = sum(1 << p for p in range(4))
TILES = {
    "256rows": mel.ENGINE_ALL | (ALL4 << 5),
    "32k": mel.ENGINE_ALL | (ALL4 << 9),
    "256rows_32k": mel.ENGINE_ALL | (ALL4 << 5) | (ALL4 << 9),
    "register_path": 0,
}


@pytest.mark.parametrize("tiles", list(TILES.values()), ids=list(TILES))
@pytest.mark.parametrize("name", ["ragged_shared_r3_s2", "wide_d320_zipf", "ragged_shared_r3_s2_f16"])
def test_merged_forward_each_tile(name, tiles):
    """The merged forward runs the streamed products without their low-rank
    pass in whichever tile build the engine word selects for gate_up and down
    (with the register path selected it still takes the default streamed
    build)."""
    require_gpu()
    ld = CASES[name]
    announce("merged tiles", f"{name} engines={tiles}", ld)
    inp = make_inputs(ld, seed=6)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    before = mel.get_engines(dims)
    mel.set_engines(dims, tiles)
    try:
        rt = mel.route(logits, dims)
        m = mel.merge_lora(w, dims)
        y_m = mel.forward_merged(x, rt, m, dims, y=torch.full_like(x, float("nan")))
        torch.cuda.synchronize()
    finally:
        mel.set_engines(dims, before)
    ids, tw = oracle.topk_softmax(inp.logits, ld.k)
    np.testing.assert_array_equal(rt.topk_ids.cpu().numpy(), ids)
    em = relerr(to_numpy_f64(y_m), oracle.forward_merged(inp, ids, tw, ld))
    print(f"merged Y {em:.2e}", flush=True)
    assert em <= TOL
