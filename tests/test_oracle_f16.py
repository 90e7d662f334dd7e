"""Pins for the oracle on fp16-element layers (CPU only).

The oracle's arithmetic is the same for both 16-bit element types; what an
fp16 layer adds is the decoding of IEEE binary16 inputs, written from the
format's definition in ``oracle.f16_decode``.  Anchors:
  * hand-decoded bit patterns (1, -2, the largest finite 65504, the smallest
    normal 2^-14, the smallest subnormal 2^-24, signed zero, 1/3 rounded,
    infinities and NaN);
  * all 65536 patterns against torch's own float16 -> float64 conversion;
  * a whole fp16 layer, forward and backward, against torch autograd on
    merged weights whose inputs torch decodes itself.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import LayerDims, make_inputs


def test_hand_decoded_patterns():
    cases = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0400: 2.0 ** -14,
             0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24, 0x3555: 0.333251953125,
             0x3C01: 1 + 2.0 ** -10, 0x7C00: np.inf, 0xFC00: -np.inf}
    bits = np.array(list(cases), np.uint16)
    got = oracle.f16_decode(bits)
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    z = oracle.f16_decode(np.array([0x0000, 0x8000], np.uint16))
    assert z[0] == 0.0 and not np.signbit(z[0]) and z[1] == 0.0 and np.signbit(z[1])
    assert np.isnan(oracle.f16_decode(np.array([0x7E00, 0xFE01], np.uint16))).all()


def test_every_pattern_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def _t16(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.float16).double()


@pytest.mark.parametrize("shared", [0, 1])
def test_fp16_layer_matches_autograd(shared):
    dims = LayerDims(T=20, d=8, n=6, E=5, k=2, r=3, n_shared=shared, lora_scale=2.0,
                     element="f16")
    inp = make_inputs(dims, seed=4, weight_std=0.3)
    ids, w = oracle.topk_softmax(inp.logits, dims.k)
    leaves = [_t16(getattr(inp, k)).requires_grad_() for k in ("x", "a_gu", "b_gu", "a_dn", "b_dn")]
    X, A_gu, B_gu, A_dn, B_dn = leaves
    W_gu, W_dn, s = _t16(inp.w_gu), _t16(inp.w_dn), dims.lora_scale
    y = torch.zeros(dims.T, dims.d, dtype=torch.float64)
    wt = torch.from_numpy(w.astype(np.float64))
    for e in range(dims.E_tot):
        if e < dims.E:
            tok, slot = np.nonzero(ids == e)
            if tok.size == 0:
                continue
            scale = wt[tok, slot][:, None]
        else:
            tok, scale = np.arange(dims.T), 1.0
        g = X[tok] @ (W_gu[e] + s * (A_gu[e] @ B_gu[e]).T).T
        gate, up = g[:, :dims.n], g[:, dims.n:]
        o = (gate * torch.sigmoid(gate) * up) @ (W_dn[e] + s * (A_dn[e] @ B_dn[e]).T).T
        y = y.index_add(0, torch.from_numpy(tok), scale * o)
    fw = oracle.forward(inp, ids, w, dims)["y"]
    assert np.max(np.abs(fw - y.detach().numpy())) <= 1e-12 * np.max(np.abs(fw))
    (y * _t16(inp.dy)).sum().backward()
    bw = oracle.backward(inp, ids, w, dims)
    for name, leaf in zip(("dx", "da_gu", "db_gu", "da_dn", "db_dn"), leaves):
        ref = leaf.grad.numpy()
        assert np.max(np.abs(bw[name] - ref)) <= 1e-11 * np.max(np.abs(ref)), name
