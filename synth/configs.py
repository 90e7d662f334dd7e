"""Layer shapes and seeded synthetic inputs.

Five workloads borrow the shapes of the models the Unsloth "faster MoE"
documentation page benchmarks (Qwen3-30B-A3B in "MoE LoRA changes things",
a 64-routed + 1-shared GLM/DeepSeek-style layer from the GLM-4.7-Flash
benchmark, and gpt-oss-20b from the gpt-oss benchmark) plus a tiny case and a
skewed-routing stress case.  No dataset or trained weight is involved: every
array is a seeded draw.

Recipe (fixed; both sides of every parity test consume exactly these arrays):

* ``numpy.random.Generator(PCG64)``; one child stream per array, spawned from
  ``SeedSequence(seed)`` in the fixed order logits, bias/popularity, x, w_gu,
  w_dn, a_gu, b_gu, a_dn, b_dn, dy.
* Normal draws are made in fp32 (``standard_normal(dtype=float32)``), scaled by
  the standard deviation in fp32 and stored as bf16 with round-to-nearest-even
  (as IEEE fp16, also round-to-nearest-even, for a layer whose element type is
  ``"f16"``; the draws are the same).
* Router logits stay fp32.  Recipes:
  ``normal``  N(0,1)  (near-uniform expert load);
  ``bias``    N(0,1) + b_e with b_e ~ N(0, 0.5) per expert;
  ``zipf``    ln p_e + Gumbel(0,1), p_e proportional to rho(e)^-1.1 for a seeded
              permutation rho of 1..E (Gumbel-top-k samples k experts without
              replacement in proportion to p, Kool et al. 2019);
  ``stress``  4 seeded hot experts always receive a token's 4 largest N(0,1)
              draws and 16 seeded empty experts its 16 smallest, so exactly half
              of all assignments land on 4 experts and 16 experts get none.
* Hidden states X ~ N(0,1); base weights, LoRA A and LoRA B ~ N(0, 0.02);
  upstream gradient dY ~ N(0,1).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

_STREAMS = ("logits", "bias", "x", "w_gu", "w_dn", "a_gu", "b_gu", "a_dn", "b_dn", "dy")


@dataclass(frozen=True)
class LayerDims:
    """Shape of one MoE-LoRA expert layer.

    T tokens, hidden size d, expert intermediate size n, E routed experts,
    top-k, LoRA rank r, n_shared always-on shared experts (0 or 1) stacked
    after the routed ones, and the LoRA scale applied to the low-rank term.
    ``element`` is the 16-bit storage type of the activations and weights:
    ``"bf16"`` or ``"f16"``.
    """

    T: int
    d: int
    n: int
    E: int
    k: int
    r: int
    n_shared: int = 0
    lora_scale: float = 1.0
    logits_recipe: str = "normal"
    name: str = field(default="custom", compare=False)
    element: str = "bf16"

    @property
    def P(self) -> int:
        """Routed (token, expert) pairs."""
        return self.T * self.k

    @property
    def P_tot(self) -> int:
        """Rows of every grouped GEMM: routed pairs plus shared-expert rows."""
        return self.T * self.k + self.n_shared * self.T

    @property
    def E_tot(self) -> int:
        return self.E + self.n_shared


CONFIGS = {
    "tiny": LayerDims(256, 128, 64, 8, 2, 4, name="tiny"),
    "qwen3_30b_a3b": LayerDims(4096, 2048, 768, 128, 8, 64, name="qwen3_30b_a3b"),
    "deepseek_shared": LayerDims(8192, 2048, 1536, 64, 4, 8, n_shared=1,
                                 logits_recipe="bias", name="deepseek_shared"),
    "long_zipf": LayerDims(16384, 2880, 2880, 32, 4, 8, logits_recipe="zipf",
                           name="long_zipf"),
    "routing_stress": LayerDims(32768, 2048, 768, 128, 8, 64, logits_recipe="stress",
                                name="routing_stress"),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Encode fp32 values as bf16 bit patterns (uint16), round to nearest even.

    The inputs are finite draws, so the NaN/overflow corner of the encoding
    never arises here.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Encode fp32 values as IEEE binary16 bit patterns (uint16), round to
    nearest even (numpy's float32 -> float16 conversion)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


_ENCODE = {"bf16": bf16_bits_from_f32, "f16": f16_bits_from_f32}


def _children(seed: int):
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(s)) for name, s in zip(_STREAMS, kids)}


def _normal16(rng: np.random.Generator, shape, std: float, element: str) -> np.ndarray:
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return _ENCODE[element](v)


def _logits(dims: LayerDims, rng: np.random.Generator, rng_b: np.random.Generator) -> np.ndarray:
    T, E = dims.T, dims.E
    recipe = dims.logits_recipe
    if recipe == "normal":
        return rng.standard_normal((T, E), dtype=np.float32)
    if recipe == "bias":
        b = rng_b.standard_normal(E, dtype=np.float32) * np.float32(0.5)
        return rng.standard_normal((T, E), dtype=np.float32) + b[None, :]
    if recipe == "zipf":
        rho = rng_b.permutation(E) + 1
        p = rho.astype(np.float64) ** -1.1
        p /= p.sum()
        g = rng.gumbel(0.0, 1.0, size=(T, E))
        return (np.log(p)[None, :] + g).astype(np.float32)
    if recipe == "stress":
        n_hot, n_empty = 4, 16
        if E < n_hot + n_empty + dims.k:
            raise ValueError("stress recipe needs E >= 20 + k")
        perm = rng_b.permutation(E)
        hot, empty, rest = perm[:n_hot], perm[n_hot:n_hot + n_empty], perm[n_hot + n_empty:]
        vals = rng.standard_normal((T, E), dtype=np.float32)
        vals.sort(axis=1)  # ascending
        out = np.empty((T, E), dtype=np.float32)
        rows = np.arange(T)[:, None]
        groups = ((empty, vals[:, :n_empty]),
                  (rest, vals[:, n_empty:E - n_hot]),
                  (hot, vals[:, E - n_hot:]))
        for experts, v in groups:
            order = np.argsort(rng.random((T, len(experts))), axis=1)
            out[rows, experts[order]] = v
        return out
    raise ValueError(f"unknown logits recipe {recipe!r}")


def make_logits(dims: LayerDims, seed: int = 0) -> np.ndarray:
    """Router logits only (same values as ``make_inputs(dims, seed).logits``)."""
    c = _children(seed)
    return _logits(dims, c["logits"], c["bias"])


@dataclass
class LayerInputs:
    """One layer's inputs; the 16-bit arrays are uint16 bit patterns of
    ``dims.element`` (bf16 or fp16).

    Layouts (row-major): logits [T,E] f32; x, dy [T,d]; w_gu [E_tot,2n,d]
    (rows [0,n) gate, [n,2n) up); w_dn [E_tot,d,n]; a_gu [E_tot,d,r];
    b_gu [E_tot,r,2n]; a_dn [E_tot,n,r]; b_dn [E_tot,r,d].
    """

    dims: LayerDims
    logits: np.ndarray
    x: np.ndarray
    w_gu: np.ndarray
    w_dn: np.ndarray
    a_gu: np.ndarray
    b_gu: np.ndarray
    a_dn: np.ndarray
    b_dn: np.ndarray
    dy: np.ndarray


def make_inputs(dims: LayerDims, seed: int = 0, weight_std: float = 0.02) -> LayerInputs:
    c = _children(seed)
    Et, d, n, r = dims.E_tot, dims.d, dims.n, dims.r
    if dims.element not in _ENCODE:
        raise ValueError(f"unknown element type {dims.element!r}")

    def _draw(rng, shape, std):
        return _normal16(rng, shape, std, dims.element)

    return LayerInputs(
        dims=dims,
        logits=_logits(dims, c["logits"], c["bias"]),
        x=_draw(c["x"], (dims.T, d), 1.0),
        w_gu=_draw(c["w_gu"], (Et, 2 * n, d), weight_std),
        w_dn=_draw(c["w_dn"], (Et, d, n), weight_std),
        a_gu=_draw(c["a_gu"], (Et, d, r), weight_std),
        b_gu=_draw(c["b_gu"], (Et, r, 2 * n), weight_std),
        a_dn=_draw(c["a_dn"], (Et, n, r), weight_std),
        b_dn=_draw(c["b_dn"], (Et, r, d), weight_std),
        dy=_draw(c["dy"], (dims.T, d), 1.0),
    )
