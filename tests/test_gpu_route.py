"""Routing on the GPU against the oracle: top-k ids, counts, offsets,
sorted_pair, pair_pos and the gather table's tokens bit-exact; routing weights
(and the gather table's weights) to fp32 rounding; NaN and infinite logits
give the oracle's ids.  The workloads, edge shapes, forced ties, non-finite
rows, and 40 seeded random shapes and logit patterns."""
import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel
import oracle
from gpu_helpers import announce, mdims, require_gpu
from synth import CONFIGS, LayerDims, make_logits

pytestmark = pytest.mark.gpu


def _run_and_compare(dims_l, logits_np):
    require_gpu()
    dims = mdims(dims_l)
    logits = torch.from_numpy(logits_np).cuda()
    out = mel.empty_routing(dims, "cuda")
    for t in out:  # sentinels: every element must be written
        t.fill_(-7)
    rt = mel.route(logits, dims, out)
    again = mel.route(logits, dims)
    torch.cuda.synchronize()
    ids, w = oracle.topk_softmax(logits_np, dims.k)
    R = oracle.route(ids, dims.E)
    tok, wgt = oracle.gather_rows(R, w, dims.T, dims.k, dims.n_shared)
    np.testing.assert_array_equal(rt.topk_ids.cpu().numpy(), ids)
    np.testing.assert_array_equal(rt.counts.cpu().numpy(), R.counts)
    np.testing.assert_array_equal(rt.offsets.cpu().numpy(), R.offsets)
    np.testing.assert_array_equal(rt.sorted_pair.cpu().numpy(), R.sorted_pair)
    np.testing.assert_array_equal(rt.pair_pos.cpu().numpy(), R.pair_pos)
    np.testing.assert_array_equal(rt.row_token.cpu().numpy(), tok)
    gw, gr = rt.topk_w.cpu().numpy(), rt.row_weight.cpu().numpy()
    fin = np.isfinite(w)
    np.testing.assert_array_equal(np.isfinite(gw), fin)
    np.testing.assert_allclose(gw[fin], w[fin], rtol=2e-6, atol=1e-7)
    np.testing.assert_array_equal(np.isfinite(gr), np.isfinite(wgt))
    # the gather table carries the same fp32 weights the GPU wrote into topk_w
    sp = R.sorted_pair.astype(np.int64)
    np.testing.assert_array_equal(gr[:dims.P], gw.reshape(-1)[sp])
    if dims.n_shared:
        assert np.all(gr[dims.P:] == 1.0)
    for a, b in zip(rt, again):  # deterministic
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("name", list(CONFIGS))
def test_route_configs(name):
    announce("route", name)
    d = CONFIGS[name]
    _run_and_compare(d, make_logits(d))


EDGE = [
    LayerDims(1, 64, 64, 5, 3, 4),        # one token
    LayerDims(100, 64, 64, 1, 1, 4),      # one expert
    LayerDims(65, 64, 64, 8, 8, 4),       # k = E, ragged last block
    LayerDims(130, 64, 64, 16, 1, 4),     # k = 1
    LayerDims(777, 64, 64, 256, 8, 4),    # widest E
    LayerDims(64, 64, 64, 256, 256, 4),   # k = E = 256
    LayerDims(1000, 64, 64, 37, 5, 4),    # E not a power of two
    LayerDims(4097, 64, 64, 16, 4, 4),    # two rounds of 16 tokens per block, ragged last block
    LayerDims(70000, 64, 64, 256, 8, 4),  # many rounds per block, several blocks per scatter group
    LayerDims(333, 64, 64, 6, 2, 4, n_shared=1),  # gather table with the shared expert's rows
    LayerDims(5000, 64, 64, 64, 4, 4, n_shared=1),
]


@pytest.mark.parametrize("dims", EDGE, ids=lambda d: f"T{d.T}E{d.E}k{d.k}")
def test_route_edges(dims):
    announce("route edge", dims)
    _run_and_compare(dims, make_logits(dims, seed=5))


def test_route_ties_and_one_hot_expert():
    announce("route ties")
    rng = np.random.default_rng(3)
    L = rng.integers(-2, 3, size=(300, 12)).astype(np.float32)
    L[::7] = 0.0  # whole rows tied
    L[5] = -0.0
    _run_and_compare(LayerDims(300, 64, 64, 12, 4, 4), L)
    L2 = np.zeros((200, 6), np.float32)
    L2[:, 4] = 3.0
    _run_and_compare(LayerDims(200, 64, 64, 6, 2, 4), L2)


def test_route_nan_and_infinite_logits():
    """Non-finite logits still give valid ids, the oracle's order (NaN below
    -inf), and a consistent grouping."""
    announce("route nan")
    rng = np.random.default_rng(12)
    L = rng.normal(size=(300, 24)).astype(np.float32)
    L[0] = np.nan
    L[1, :20] = np.nan
    L[2, [3, 7]] = -np.inf
    L[2, [1, 5]] = np.nan
    L[3, 4] = np.inf
    L[4, ::2] = np.nan
    L[5] = -np.inf
    L[17::23, 5] = np.nan
    _run_and_compare(LayerDims(300, 64, 64, 24, 6, 4), L)


def _random_route_case(i: int):
    """Routing shape and logits of case i (fixed by i alone): T up to 40000,
    E up to 256, k up to min(E, 16), the shared expert, a logit recipe, and
    in some cases ties (logits rounded to a coarse grid) or non-finite values."""
    g = np.random.default_rng(9000 + i)
    E = int(g.choice([1, 2, 3, 7, 16, 31, 64, 100, 128, 200, 256]))
    k = int(g.integers(1, min(E, 16) + 1))
    recipes = ["normal", "bias", "zipf"] + (["stress"] if E >= 20 + k else [])
    ld = LayerDims(T=int(g.choice([1, 5, 16, 17, 255, 1000, 4096, 9999, 40000])), d=64, n=64, E=E,
                   k=k, r=4, n_shared=int(g.integers(0, 2)), logits_recipe=str(g.choice(recipes)))
    L = make_logits(ld, seed=i)
    mode = int(g.integers(0, 4))
    if mode == 1:  # ties: many equal logits within a row
        L = np.round(L * 2.0) / 2.0
    elif mode == 2:  # scattered non-finite logits
        m = g.random(L.shape)
        L[m < 0.01] = np.nan
        L[(m >= 0.01) & (m < 0.015)] = np.inf
        L[(m >= 0.015) & (m < 0.02)] = -np.inf
    return ld, L.astype(np.float32)


@pytest.mark.parametrize("i", range(40))
def test_route_random(i):
    ld, L = _random_route_case(i)
    announce("route random", i, ld)
    _run_and_compare(ld, L)
