"""Parity over seeded random layer shapes: every case draws T, d, n, E, k, r,
the shared expert, the LoRA scale, the logit recipe, the element type and an
engine/tile setting inside the library's envelope, then runs route + forward
+ backward (router gradients included) on the GPU and compares every output
with the float64 oracle built from the oracle's own routing (top-k ids bit
for bit).  The draws are fixed by the case number, so a failing case can be
run again by its id."""

import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel
import oracle
from gpu_helpers import TOL, announce, compare_layer, mdims, require_gpu, to_numpy_f64, upload
from synth import LayerDims, make_inputs

pytestmark = pytest.mark.gpu

ALL4 = sum(1 << p for p in range(4))


def _engine_words():
    return [0, mel.ENGINE_ALL, mel.ENGINE_ALL | (ALL4 << 5), mel.ENGINE_ALL | (ALL4 << 9),
            mel.ENGINE_ALL | (ALL4 << 5) | (ALL4 << 9), mel.ENGINE_ALL | mel.SPLITK_1024,
            mel.ENGINE_ALL | mel.SPLITK_4096,
            mel.ENGINE_GATE_UP | mel.ENGINE_DX | mel.ENGINE_RANK | mel.TILE256(3) | mel.STAGE32(0)]


def draw_case(i: int):
    """Layer shape and engine word of case i (fixed by i alone)."""
    g = np.random.default_rng(1000 + i)
    E = int(g.integers(1, 41))
    k = int(g.integers(1, min(E, 8) + 1))
    recipes = ["normal", "bias", "zipf"] + (["stress"] if E >= 20 + k else [])
    ld = LayerDims(
        T=int(g.choice([1, 2, 3, 17, 64, 129, 333, 600])),
        d=64 * int(g.integers(1, 9)),
        n=64 * int(g.integers(1, 9)),
        E=E, k=k,
        r=int(g.choice([1, 2, 5, 8, 13, 16, 31, 64, 100, 128])),
        n_shared=int(g.integers(0, 2)),
        lora_scale=float(g.choice([1.0, 2.0, 0.5, -1.5])),
        logits_recipe=str(g.choice(recipes)),
        element=str(g.choice(["bf16", "f16"])),
    )
    words = _engine_words()
    return ld, words[int(g.integers(0, len(words)))]


N_CASES = 48


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_parity(i):
    require_gpu()
    ld, engines = draw_case(i)
    announce("random", i, f"engines={engines}", ld)
    inp = make_inputs(ld, seed=i)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    before = mel.get_engines(dims)
    mel.set_engines(dims, engines)
    try:
        layer = mel.MoELoRALayer(dims, w)
        layer.y.fill_(float("nan"))
        for t in layer.grads:
            t.fill_(float("nan"))
        layer.route(logits)
        y = layer.forward(x)
        g = layer.backward(dy, x, router=True)
        torch.cuda.synchronize()
    finally:
        mel.set_engines(dims, before)
    ids, tw = oracle.topk_softmax(inp.logits, ld.k)
    np.testing.assert_array_equal(layer.routing.topk_ids.cpu().numpy(), ids)
    np.testing.assert_allclose(layer.routing.topk_w.cpu().numpy(), tw, rtol=2e-6, atol=1e-7)
    fw = oracle.forward(inp, ids, tw, ld)
    bw = oracle.backward(inp, ids, tw, ld)
    rgr = oracle.router_grads(inp, ids, tw, ld, fw=fw)
    rg = layer.router_grads
    got = {"y": y, "dx": g.dx, "da_gu": g.da_gate_up, "db_gu": g.db_gate_up,
           "da_dn": g.da_down, "db_dn": g.db_down, "d_topk_w": rg.d_topk_w, "d_logits": rg.d_logits}
    errs = compare_layer(got, fw, bw, rgr)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for key, e in errs.items():
        assert e <= TOL, (key, e)
    counts = np.bincount(ids.reshape(-1), minlength=ld.E)
    for e in np.nonzero(counts == 0)[0]:
        for key in ("da_gu", "db_gu", "da_dn", "db_dn"):
            assert not np.any(to_numpy_f64(got[key])[e]), (key, e)


def draw_medium(i: int):
    """A larger layer for case i of the second group: segments of several
    tiles and split-K chunks (fixed by i alone)."""
    g = np.random.default_rng(5000 + i)
    E = int(g.integers(2, 131))
    k = int(g.integers(1, min(E, 8) + 1))
    recipes = ["normal", "bias", "zipf"] + (["stress"] if E >= 20 + k else [])
    ld = LayerDims(
        T=int(g.integers(700, 3001)),
        d=64 * int(g.integers(1, 13)),
        n=64 * int(g.integers(1, 13)),
        E=E, k=k,
        r=int(g.choice([3, 8, 16, 24, 64, 128])),
        n_shared=int(g.integers(0, 2)),
        lora_scale=float(g.choice([1.0, 2.0, 0.5])),
        logits_recipe=str(g.choice(recipes)),
        element=str(g.choice(["bf16", "f16"])),
    )
    words = _engine_words()
    return ld, words[int(g.integers(0, len(words)))]


N_MEDIUM = 16


@pytest.mark.parametrize("i", range(N_MEDIUM))
def test_random_medium_shape_parity(i):
    """As above on larger layers, against the float32 oracle."""
    require_gpu()
    ld, engines = draw_medium(i)
    announce("random medium", i, f"engines={engines}", ld)
    inp = make_inputs(ld, seed=100 + i)
    dims = mdims(ld)
    logits, x, dy, w = upload(inp)
    before = mel.get_engines(dims)
    mel.set_engines(dims, engines)
    try:
        layer = mel.MoELoRALayer(dims, w)
        layer.y.fill_(float("nan"))
        for t in layer.grads:
            t.fill_(float("nan"))
        layer.route(logits)
        y = layer.forward(x)
        g = layer.backward(dy, x, router=True)
        torch.cuda.synchronize()
    finally:
        mel.set_engines(dims, before)
    ids, tw = oracle.topk_softmax(inp.logits, ld.k)
    np.testing.assert_array_equal(layer.routing.topk_ids.cpu().numpy(), ids)
    f32 = np.float32
    fw = oracle.forward(inp, ids, tw, ld, dtype=f32)
    bw = oracle.backward(inp, ids, tw, ld, dtype=f32)
    rgr = oracle.router_grads(inp, ids, tw, ld, dtype=f32, fw=fw)
    rg = layer.router_grads
    got = {"y": y, "dx": g.dx, "da_gu": g.da_gate_up, "db_gu": g.db_gate_up,
           "da_dn": g.da_down, "db_dn": g.db_down, "d_topk_w": rg.d_topk_w, "d_logits": rg.d_logits}
    errs = compare_layer(got, fw, bw, rgr)
    print("errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for key, e in errs.items():
        assert e <= TOL, (key, e)
