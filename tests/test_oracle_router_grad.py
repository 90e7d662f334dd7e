"""Pins for the oracle's router gradients (CPU only).

``oracle.router_grads`` gives d_topk_w = <dY, O_pair> and the logit gradient
through the softmax over the k selected logits.  Anchors, none of which
re-types those two formulas:
  * central differences of L = <dY, Y> through the oracle's whole forward,
    perturbing one routing weight at a time (Y is linear in the weights, so
    the difference quotient is exact up to float64 rounding);
  * central differences of L through the routing itself: the k selected
    logits go through a float64 softmax written here, the weights into the
    oracle's forward, the selection held fixed (it is, for these steps);
  * k = E (softmax over every expert) against torch.autograd;
  * k = 1 (weight fixed at 1): every logit gradient is exactly 0;
  * the logit gradient of each token sums to 0 up to the float32 rounding of
    the weights (adding a constant to every logit leaves the softmax
    unchanged) and is exactly 0 off the selection.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import LayerDims, make_inputs


def _dims(**kw):
    base = dict(T=12, d=16, n=8, E=6, k=3, r=4, n_shared=0, lora_scale=1.0)
    base.update(kw)
    return LayerDims(**base)


def _loss(inp, ids, w, dims):
    y = oracle.forward(inp, ids, w, dims)["y"]
    return float(np.sum(oracle.bf16_decode(inp.dy) * y))


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("shared", [0, 1])
def test_d_topk_w_is_the_weight_derivative_of_the_loss(shared):
    dims = _dims(n_shared=shared)
    inp = make_inputs(dims, seed=3)
    ids, w = oracle.topk_softmax(inp.logits, dims.k)
    g = oracle.router_grads(inp, ids, w, dims)["d_topk_w"]
    rng = np.random.default_rng(0)
    for t, j in zip(rng.integers(0, dims.T, 8), rng.integers(0, dims.k, 8)):
        wp, wm = w.copy(), w.copy()
        wp[t, j] = np.float32(w[t, j] + 0.25)
        wm[t, j] = np.float32(w[t, j] - 0.25)
        step = float(wp[t, j]) - float(wm[t, j])  # exact in float64
        fd = (_loss(inp, ids, wp, dims) - _loss(inp, ids, wm, dims)) / step
        assert abs(fd - g[t, j]) <= 1e-9 * max(1.0, abs(g[t, j]))


def _softmax64(v):
    e = np.exp(v - v.max())
    return e / e.sum()


def test_d_logits_matches_differences_through_the_routing():
    dims = _dims()
    inp = make_inputs(dims, seed=5)
    ids, w = oracle.topk_softmax(inp.logits, dims.k)
    dl = oracle.router_grads(inp, ids, w, dims)["d_logits"]
    logits = inp.logits.astype(np.float64)

    def loss_at(lg):
        # float64 softmax over the (fixed) selection, weights into the forward
        ww = np.stack([_softmax64(lg[t, ids[t]]) for t in range(dims.T)])
        # forward rounds weights to float32: linear in w, so evaluate the loss
        # as sum_j w_j <dY, O_j> with the oracle's own per-pair outputs
        return float(np.sum(ww * c))

    o = oracle.forward(inp, ids, w, dims)["o_pair"][: dims.T * dims.k].reshape(dims.T, dims.k, dims.d)
    c = np.einsum("tc,tjc->tj", oracle.bf16_decode(inp.dy), o)
    eps = 1e-5
    rng = np.random.default_rng(1)
    for t in rng.integers(0, dims.T, 6):
        for e in range(dims.E):
            lp, lm = logits.copy(), logits.copy()
            lp[t, e] += eps
            lm[t, e] -= eps
            # the steps do not change the selection
            assert (oracle.topk_softmax(lp.astype(np.float32), dims.k)[0][t] == ids[t]).all() or e not in ids[t]
            fd = (loss_at(lp) - loss_at(lm)) / (2 * eps) if e in ids[t] else 0.0
            assert abs(fd - dl[t, e]) <= 1e-6 * max(1.0, np.max(np.abs(dl)))
    # every unselected logit is exactly 0, every row sums to 0
    mask = np.zeros_like(dl, bool)
    mask[np.arange(dims.T)[:, None], ids.astype(np.int64)] = True
    assert np.all(dl[~mask] == 0.0)
    # (exactly 0 for weights summing to 1; the weights are float32)
    dw = oracle.router_grads(inp, ids, w, dims)["d_topk_w"]
    assert np.max(np.abs(dl.sum(axis=1))) <= 1e-6 * np.max(np.abs(dw))


def test_k_equals_E_matches_autograd():
    dims = _dims(E=4, k=4)
    inp = make_inputs(dims, seed=7)
    ids, w = oracle.topk_softmax(inp.logits, dims.k)
    got = oracle.router_grads(inp, ids, w, dims)
    o = oracle.forward(inp, ids, w, dims)["o_pair"][: dims.T * dims.k].reshape(dims.T, dims.k, dims.d)
    # per-expert outputs in expert order, then y = softmax(logits) . O
    oe = np.zeros((dims.T, dims.E, dims.d))
    oe[np.arange(dims.T)[:, None], ids.astype(np.int64)] = o
    lg = torch.tensor(inp.logits.astype(np.float64), requires_grad=True)
    y = torch.einsum("te,tec->tc", torch.softmax(lg, dim=1), torch.tensor(oe))
    (y * torch.tensor(oracle.bf16_decode(inp.dy))).sum().backward()
    assert np.max(np.abs(lg.grad.numpy() - got["d_logits"])) <= 1e-6 * np.max(np.abs(got["d_logits"]))


def test_k_one_has_no_logit_gradient():
    dims = _dims(k=1)
    inp = make_inputs(dims, seed=9)
    ids, w = oracle.topk_softmax(inp.logits, dims.k)
    got = oracle.router_grads(inp, ids, w, dims)
    assert np.all(w == 1.0)
    assert np.all(got["d_logits"] == 0.0)
    assert np.max(np.abs(got["d_topk_w"])) > 0


def test_token_rows_match_the_whole_batch():
    dims = _dims(n_shared=1)
    inp = make_inputs(dims, seed=11)
    ids, w = oracle.topk_softmax(inp.logits, dims.k)
    full = oracle.router_grads(inp, ids, w, dims)
    toks = [0, 5, dims.T - 1]
    rows = oracle.router_grads_tokens(inp, ids, w, dims, toks)
    for key in ("d_topk_w", "d_logits"):
        assert np.max(np.abs(rows[key] - full[key][toks])) <= 1e-12 * np.max(np.abs(full[key]))
