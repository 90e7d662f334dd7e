"""Pins for the oracle's expert MLP, combine and backward (CPU only).

Anchors, none of which re-types the oracle's own formulas:
  * a hand-worked 2-dim example whose outputs and gradients are written out as
    scalar closed forms (catches a dropped LoRA term, a wrong sign, a swapped
    gate/up half, a transposed non-square operand);
  * split LoRA equal to the merged-weight path W + s (A B)^T in float64 --
    the identity the Unsloth "faster MoE" page rests on ("Faster LoRA MoE
    training");
  * the sorted grouping equal to the per-expert search loop;
  * special cases that reduce to library routines (torch.nn.functional on a
    dense MLP, torch.softmax for k = E, B = 0 for a plain MoE);
  * torch.autograd on an independently written merged-weight layer, and
    central finite differences, for every gradient;
  * parameter counts the page prints ("MoE LoRA changes things",
    "Implementation details"), from tests/golden/page_numbers.json.
"""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import CONFIGS, LayerDims, LayerInputs, bf16_bits_from_f32, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _routing(inp):
    return oracle.topk_softmax(inp.logits, inp.dims.k)


def _small(**kw):
    base = dict(T=24, d=8, n=6, E=5, k=2, r=3, n_shared=0, lora_scale=1.0)
    base.update(kw)
    return LayerDims(**base)


def _f(a):
    return oracle.bf16_decode(a)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- hand example

def _b(v):
    return bf16_bits_from_f32(np.asarray(v, np.float32))


def _hand_inputs():
    """T=1, E=2, k=1, d=2, n=1, r=1, s=1; the token is routed to expert 1."""
    dims = LayerDims(1, 2, 1, 2, 1, 1)
    three = np.full((1,), 3.0, np.float32)
    inp = LayerInputs(
        dims=dims,
        logits=np.array([[0.0, 1.0]], np.float32),
        x=_b([[1.0, 2.0]]),
        w_gu=_b([np.full((2, 2), 3.0), [[1.0, 0.5], [0.25, 1.0]]]),   # [E, 2n, d]
        w_dn=_b([np.full((2, 1), 3.0), [[1.0], [2.0]]]),              # [E, d, n]
        a_gu=_b([np.full((2, 1), 3.0), [[1.0], [1.0]]]),              # [E, d, r]
        b_gu=_b([np.full((1, 2), 3.0), [[0.5, -0.25]]]),              # [E, r, 2n]
        a_dn=_b([three.reshape(1, 1), [[2.0]]]),                      # [E, n, r]
        b_dn=_b([np.full((1, 2), 3.0), [[1.0, 0.0]]]),                # [E, r, d]
        dy=_b([[1.0, -1.0]]),
    )
    return inp


def test_hand_worked_example():
    inp = _hand_inputs()
    ids, w = _routing(inp)
    assert ids.tolist() == [[1]] and w.tolist() == [[1.0]]
    # gate = 1*1 + 2*0.5 = 2, up = 1*0.25 + 2*1 = 2.25, X A = 3,
    # LoRA adds 3 * [0.5, -0.25]  ->  G = [3.5, 1.5]
    sig = 1.0 / (1.0 + math.exp(-3.5))
    h = 3.5 * sig * 1.5
    # O = W_dn h + (h A_dn) B_dn = [h, 2h] + [2h, 0]
    y_expect = np.array([[3.0 * h, 2.0 * h]])
    fw = oracle.forward(inp, ids, w, inp.dims, keep=True)
    np.testing.assert_allclose(fw["g"], [[3.5, 1.5]], rtol=1e-15)
    np.testing.assert_allclose(fw["xa"], [[3.0]], rtol=1e-15)
    np.testing.assert_allclose(fw["ha"], [[2.0 * h]], rtol=1e-15)
    np.testing.assert_allclose(fw["y"], y_expect, rtol=1e-14)
    # backward with dY = [1, -1]:
    # q_dn = 1, dH = (1 - 2) + 2 = 1
    dgate = 1.5 * sig * (1.0 + 3.5 * (1.0 - sig))
    dup = 3.5 * sig
    q_gu = 0.5 * dgate - 0.25 * dup
    bw = oracle.backward(inp, ids, w, inp.dims)
    np.testing.assert_allclose(bw["dx"], [[dgate + 0.25 * dup + q_gu, 0.5 * dgate + dup + q_gu]],
                               rtol=1e-14)
    np.testing.assert_allclose(bw["db_dn"][1], [[2.0 * h, -2.0 * h]], rtol=1e-14)
    np.testing.assert_allclose(bw["da_dn"][1], [[h]], rtol=1e-14)
    np.testing.assert_allclose(bw["db_gu"][1], [[3.0 * dgate, 3.0 * dup]], rtol=1e-14)
    np.testing.assert_allclose(bw["da_gu"][1], [[q_gu], [2.0 * q_gu]], rtol=1e-14)
    for key in ("da_gu", "db_gu", "da_dn", "db_dn"):
        assert not np.any(bw[key][0])  # expert 0 received nothing


@pytest.mark.parametrize("s", [1.0, 2.0])
def test_hand_merged_weights(s):
    """W' = W + s (A B)^T written out for the hand example's experts."""
    inp = _hand_inputs()
    dims = replace(inp.dims, lora_scale=s)
    wgu, wdn = oracle.merged_weights(replace(inp, dims=dims), dims)
    # expert 1: A_gu B_gu = [[0.5, -0.25], [0.5, -0.25]] ([d, 2n]); its
    # transpose is added to W_gu [[1, 0.5], [0.25, 1]] ([2n, d])
    np.testing.assert_array_equal(wgu[1], [[1.0 + 0.5 * s, 0.5 + 0.5 * s],
                                           [0.25 - 0.25 * s, 1.0 - 0.25 * s]])
    # A_dn B_dn = [[2, 0]] ([n, d]); transposed onto W_dn [[1], [2]] ([d, n])
    np.testing.assert_array_equal(wdn[1], [[1.0 + 2.0 * s], [2.0]])
    # expert 0: every entry 3, so each delta entry is 3 * 3 (r = 1)
    np.testing.assert_array_equal(wgu[0], np.full((2, 2), 3.0 + 9.0 * s))
    np.testing.assert_array_equal(wdn[0], np.full((2, 1), 3.0 + 9.0 * s))
    # at s = 1 the merged gate_up row gives the G of the hand example
    if s == 1.0:
        np.testing.assert_array_equal(np.array([1.0, 2.0]) @ wgu[1].T, [3.5, 1.5])


def test_hand_combine_and_shared_expert():
    """Two routed experts with weights 3/4 and 1/4 plus a shared expert."""
    dims = LayerDims(1, 2, 1, 2, 2, 1, n_shared=1)
    # every expert: gate = x0 * a_e, up = x1; LoRA B = 0; O = [h, 0]
    a = [1.0, 2.0, 0.5]
    inp = LayerInputs(
        dims=dims,
        logits=np.array([[0.0, math.log(3.0)]], np.float32),
        x=_b([[1.0, 1.0]]),
        w_gu=_b([[[ae, 0.0], [0.0, 1.0]] for ae in a]),
        w_dn=_b([[[1.0], [0.0]]] * 3),
        a_gu=_b(np.ones((3, 2, 1))), b_gu=_b(np.zeros((3, 1, 2))),
        a_dn=_b(np.ones((3, 1, 1))), b_dn=_b(np.zeros((3, 1, 2))),
        dy=_b([[1.0, 1.0]]),
    )
    ids, w = _routing(inp)
    assert ids.tolist() == [[1, 0]]
    np.testing.assert_allclose(w, [[0.75, 0.25]], rtol=1e-6)
    silu = lambda v: v / (1.0 + math.exp(-v))
    y0 = float(w[0, 0]) * silu(2.0) + float(w[0, 1]) * silu(1.0) + silu(0.5)
    y = oracle.forward(inp, ids, w, dims)["y"]
    np.testing.assert_allclose(y, [[y0, 0.0]], rtol=1e-14, atol=0)


# ---------------------------------------------------------------- identities

@pytest.mark.parametrize("dims", [_small(), _small(n_shared=1, lora_scale=2.0),
                                  _small(k=5, E=5), CONFIGS["tiny"]])
def test_split_equals_merged_and_naive(dims):
    inp = make_inputs(dims, seed=7, weight_std=0.3)
    ids, w = _routing(inp)
    y = oracle.forward(inp, ids, w, dims)["y"]
    assert _rel(oracle.forward_merged(inp, ids, w, dims), y) <= 1e-12
    assert _rel(oracle.forward_naive(inp, ids, w, dims), y) <= 1e-12
    toks = [0, dims.T // 2, dims.T - 1]
    assert _rel(oracle.forward_tokens(inp, ids, w, dims, toks), y[toks]) <= 1e-12
    yf = oracle.forward(inp, ids, w, dims, dtype=np.float32)["y"]
    assert _rel(yf, y) <= 1e-5


def _torch_mlp(x, e, W, s):
    """Dense SwiGLU MLP with unmerged LoRA, written with torch.nn.functional."""
    g = F.linear(x, W["w_gu"][e]) + s * F.linear(F.linear(x, W["a_gu"][e].T), W["b_gu"][e].T)
    gate, up = g.chunk(2, dim=-1)
    h = F.silu(gate) * up
    return F.linear(h, W["w_dn"][e]) + s * F.linear(F.linear(h, W["a_dn"][e].T), W["b_dn"][e].T)


def _torch_params(inp):
    return {k: torch.from_numpy(_f(getattr(inp, k))) for k in
            ("w_gu", "w_dn", "a_gu", "b_gu", "a_dn", "b_dn")}


def test_single_expert_is_dense_mlp():
    dims = _small(E=1, k=1)
    inp = make_inputs(dims, seed=2, weight_std=0.3)
    ids, w = _routing(inp)
    assert np.all(w == 1.0)
    ref = _torch_mlp(torch.from_numpy(_f(inp.x)), 0, _torch_params(inp), dims.lora_scale).numpy()
    assert _rel(oracle.forward(inp, ids, w, dims)["y"], ref) <= 1e-12


def test_k_equals_E_is_dense_softmax_mixture():
    dims = _small(E=4, k=4, n_shared=1)
    inp = make_inputs(dims, seed=4, weight_std=0.3)
    ids, w = _routing(inp)
    x = torch.from_numpy(_f(inp.x))
    W = _torch_params(inp)
    p = torch.softmax(torch.from_numpy(inp.logits).double(), dim=1)
    ref = sum(p[:, e:e + 1] * _torch_mlp(x, e, W, 1.0) for e in range(4)) + _torch_mlp(x, 4, W, 1.0)
    assert _rel(oracle.forward(inp, ids, w, dims)["y"], ref.numpy()) <= 1e-6


def test_zero_B_is_plain_moe_and_G_linear_in_scale():
    dims = _small()
    inp = make_inputs(dims, seed=5, weight_std=0.3)
    ids, w = _routing(inp)
    plain = replace(inp, b_gu=np.zeros_like(inp.b_gu), b_dn=np.zeros_like(inp.b_dn))
    x = torch.from_numpy(_f(inp.x))
    W = _torch_params(plain)
    y_ref = np.zeros((dims.T, dims.d))
    for t in range(dims.T):
        for j in range(dims.k):
            e = int(ids[t, j])
            gate = F.linear(x[t], W["w_gu"][e][:dims.n])
            up = F.linear(x[t], W["w_gu"][e][dims.n:])
            y_ref[t] += float(w[t, j]) * F.linear(F.silu(gate) * up, W["w_dn"][e]).numpy()
    assert _rel(oracle.forward(plain, ids, w, dims)["y"], y_ref) <= 1e-12
    # the pre-activation is affine in the LoRA scale
    g = {s: oracle.forward(inp, ids, w, replace(dims, lora_scale=s), keep=True)["g"] for s in (0.0, 1.0, 2.5)}
    np.testing.assert_allclose(g[2.5], g[0.0] + 2.5 * (g[1.0] - g[0.0]), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- gradients

def _torch_layer_merged(inp, ids, w, dims, X, A_gu, B_gu, A_dn, B_dn):
    """Autograd reference on merged weights W + s (A B)^T (never split)."""
    s = dims.lora_scale
    W_gu = torch.from_numpy(_f(inp.w_gu))
    W_dn = torch.from_numpy(_f(inp.w_dn))
    y = torch.zeros(dims.T, dims.d, dtype=torch.float64)
    wt = torch.from_numpy(w.astype(np.float64))
    for e in range(dims.E_tot):
        wgu = W_gu[e] + s * (A_gu[e] @ B_gu[e]).T
        wdn = W_dn[e] + s * (A_dn[e] @ B_dn[e]).T
        if e < dims.E:
            tok, slot = np.nonzero(ids == e)
            if tok.size == 0:
                continue
            scale = wt[tok, slot][:, None]
        else:
            tok, scale = np.arange(dims.T), 1.0
        g = X[tok] @ wgu.T
        gate, up = g[:, :dims.n], g[:, dims.n:]
        o = (gate * torch.sigmoid(gate) * up) @ wdn.T
        y = y.index_add(0, torch.from_numpy(tok), scale * o)
    return y


@pytest.mark.parametrize("dims", [_small(), _small(n_shared=1, lora_scale=2.0),
                                  _small(E=28, k=6, T=30, logits_recipe="stress")])
def test_backward_matches_autograd(dims):
    inp = make_inputs(dims, seed=11, weight_std=0.3)
    ids, w = _routing(inp)
    leaves = [torch.from_numpy(_f(getattr(inp, k)).copy()).requires_grad_()
              for k in ("x", "a_gu", "b_gu", "a_dn", "b_dn")]
    y = _torch_layer_merged(inp, ids, w, dims, *leaves)
    (y * torch.from_numpy(_f(inp.dy))).sum().backward()
    bw = oracle.backward(inp, ids, w, dims)
    for name, leaf in zip(("dx", "da_gu", "db_gu", "da_dn", "db_dn"), leaves):
        assert _rel(bw[name], leaf.grad.numpy()) <= 1e-11, name
    if dims.logits_recipe == "stress":
        empty = np.bincount(ids.reshape(-1), minlength=dims.E) == 0
        assert empty.sum() == 16
        for key in ("da_gu", "db_gu", "da_dn", "db_dn"):
            assert not np.any(bw[key][empty])
    toks = [1, dims.T - 2]
    assert _rel(oracle.backward_tokens(inp, ids, w, dims, toks), bw["dx"][toks]) <= 1e-12
    for e in (0, dims.E_tot - 1):
        for name, got in zip(("da_gu", "db_gu", "da_dn", "db_dn"),
                             oracle.lora_grads_expert(inp, ids, w, dims, e)):
            np.testing.assert_allclose(got, bw[name][e], rtol=1e-12, atol=1e-14)


def test_backward_finite_differences():
    dims = _small(T=12, d=6, n=4, E=4, k=2, r=2, n_shared=1, lora_scale=1.5)
    inp = make_inputs(dims, seed=13, weight_std=0.3)
    ids, w = _routing(inp)
    R = _f(inp.dy)
    floats = {k: _f(getattr(inp, k)).copy() for k in
              ("x", "w_gu", "w_dn", "a_gu", "b_gu", "a_dn", "b_dn")}

    def loss(fl):
        probe = replace(inp, **fl)
        return float(np.sum(oracle.forward(probe, ids, w, dims)["y"] * R))

    bw = oracle.backward(replace(inp, **floats), ids, w, dims)
    rng = np.random.default_rng(0)
    for name, gname in (("x", "dx"), ("a_gu", "da_gu"), ("b_gu", "db_gu"),
                        ("a_dn", "da_dn"), ("b_dn", "db_dn")):
        arr = floats[name]
        for flat in rng.choice(arr.size, size=min(64, arr.size), replace=False):
            idx = np.unravel_index(flat, arr.shape)
            h = 1e-6 * max(1.0, abs(arr[idx]))
            plus, minus = dict(floats), dict(floats)
            plus[name] = arr.copy(); plus[name][idx] += h
            minus[name] = arr.copy(); minus[name][idx] -= h
            fd = (loss(plus) - loss(minus)) / (2 * h)
            g = bw[gname][idx]
            assert abs(fd - g) <= 1e-6 * max(1.0, abs(g)), (name, idx, fd, g)


# ---------------------------------------------------------------- printed numbers

def test_page_parameter_counts():
    gold = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))
    q = gold["lora_params_per_projection_qwen3_30b_a3b"]
    dims = CONFIGS["qwen3_30b_a3b"]
    assert (dims.d, dims.n, dims.r, dims.E, dims.k) == tuple(q["shapes"][c] for c in "mnrEk")
    # one down-projection adapter of the storage layout: A_dn [n, r] + B_dn [r, d]
    per_expert = dims.n * dims.r + dims.r * dims.d
    assert per_expert == q["value"]
    frac = 100.0 * per_expert / (dims.d * dims.n)
    assert abs(frac - gold["lora_params_fraction_qwen3_30b_a3b"]["value_percent_approx"]) < 0.5
    t = gold["lora_params_typical_mlp"]
    m, n, r = (t["shapes"][c] for c in "mnr")
    lora, full = m * r + r * n, m * n
    assert abs(lora - t["lora_approx"]) / t["lora_approx"] < 0.05
    assert abs(full - t["full_approx"]) / t["full_approx"] < 0.05
    assert abs(100.0 * lora / full - t["percent_approx"]) < 0.2
    # memory crossover: E*m*n (merged delta) > k*s*n (split) while s < E*m/k
    assert dims.E * dims.d // dims.k == gold["memory_crossover_tokens"]["value"]
