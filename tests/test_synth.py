"""The seeded input generator: reproducible, and its bf16 and fp16 encodings
are round-to-nearest-even (checked against torch's own float32 casts)."""
import numpy as np
import torch

from synth import CONFIGS, LayerDims, bf16_bits_from_f32, f16_bits_from_f32, make_inputs, make_logits


def test_bf16_encoding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1e-40, -3e38], np.float32)])
    ours = bf16_bits_from_f32(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_reproducible_and_seed_dependent():
    a = make_inputs(CONFIGS["tiny"], seed=0)
    b = make_inputs(CONFIGS["tiny"], seed=0)
    c = make_inputs(CONFIGS["tiny"], seed=1)
    for name in ("logits", "x", "w_gu", "w_dn", "a_gu", "b_gu", "a_dn", "b_dn", "dy"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
        assert not np.array_equal(getattr(a, name), getattr(c, name))
    np.testing.assert_array_equal(make_logits(CONFIGS["tiny"]), a.logits)


def test_shapes_and_scales():
    dims = LayerDims(64, 128, 64, 8, 2, 4, n_shared=1)
    inp = make_inputs(dims)
    Et = dims.E_tot
    assert inp.w_gu.shape == (Et, 128, 128) and inp.w_dn.shape == (Et, 128, 64)
    assert inp.a_gu.shape == (Et, 128, 4) and inp.b_gu.shape == (Et, 4, 128)
    assert inp.a_dn.shape == (Et, 64, 4) and inp.b_dn.shape == (Et, 4, 128)
    w = (inp.w_gu.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(w.std()) - 0.02) < 0.002
    x = (inp.x.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(x.std()) - 1.0) < 0.05


def test_f16_encoding_matches_torch_and_keeps_the_draws():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -25,
                                  3 * 2 ** -26, 65504.0, -6.1e-5], np.float32)])
    ours = f16_bits_from_f32(v)
    ref = torch.from_numpy(v).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # an fp16 layer draws the same normals as its bf16 twin, only stored differently
    bf = make_inputs(LayerDims(16, 64, 32, 4, 2, 4), seed=3)
    hf = make_inputs(LayerDims(16, 64, 32, 4, 2, 4, element="f16"), seed=3)
    xb = (bf.x.astype(np.uint32) << 16).view(np.float32)
    xh = hf.x.view(np.float16).astype(np.float32)
    assert np.max(np.abs(xb - xh)) <= 2 ** -8 * np.max(np.abs(xb))
    np.testing.assert_array_equal(bf.logits, hf.logits)
