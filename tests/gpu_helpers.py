"""Helpers shared by the GPU parity tests: upload seeded inputs, call the HIP
library through its binding, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import mixture_experts_lora_amd as mel

TOL = 2e-2  # max |gpu - ref| / max |ref| per tensor (16-bit inputs, fp32 accumulate)


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mel.load()  # the HIP library must be there: no fallback


def announce(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


ELEMENT = {"bf16": (mel.MOE_BF16, torch.bfloat16), "f16": (mel.MOE_F16, torch.float16)}


def mdims(ld) -> mel.Dims:
    return mel.Dims(ld.T, ld.d, ld.n, ld.E, ld.k, ld.r, ld.n_shared, ld.lora_scale,
                    ELEMENT[ld.element][0])


def elem_tensor(bits: np.ndarray, dev="cuda", element: str = "bf16") -> torch.Tensor:
    """uint16 bit patterns of the given element type -> a GPU tensor of it."""
    return torch.from_numpy(bits.view(np.int16)).to(dev).view(ELEMENT[element][1])


def to_numpy_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def upload(inp, dev="cuda"):
    el = inp.dims.element
    w = mel.Weights(*(elem_tensor(getattr(inp, k), dev, el) for k in
                      ("w_gu", "w_dn", "a_gu", "b_gu", "a_dn", "b_dn")))
    logits = torch.from_numpy(inp.logits).to(dev)
    return logits, elem_tensor(inp.x, dev, el), elem_tensor(inp.dy, dev, el), w


def relerr(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref))
    if scale == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / scale)


# Floor of the per-expert normaliser, as a fraction of the whole tensor's
# largest reference value.  The adapter gradients contract the layer's rank-r
# rows (s X A_gu, s H A_dn, Q_gu, Q_dn), dot products that the method keeps
# in 16 bits; their rounding error is relative to the dot product's terms, not
# to its sum.  When an expert's few rows give a nearly cancelling sum, its
# whole slice is tiny against an error its terms set (seeded random case 29 of
# test_gpu_random_shapes: a T = 1, r = 1 expert whose Q_gu cancels 43-fold
# has 19 % error against its own slice, exactly what rounding the same
# intermediates to bf16 on the CPU gives).  Slices of at least this fraction
# of the tensor keep their own normaliser; smaller ones are still held ten
# times tighter than the per-tensor bound.
EXPERT_FLOOR = 0.1


def relerr_per_expert(got, ref) -> float:
    """The largest per-expert error of an [E_tot, ...] gradient, each expert's
    slice normalised by its own largest reference value (a lightly loaded
    expert's error is not hidden under a hot expert's magnitude), but never by
    less than EXPERT_FLOOR times the tensor's.  An expert whose reference is
    all zero (no rows) must be exactly zero."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    floor = EXPERT_FLOOR * float(np.max(np.abs(ref)))
    worst = 0.0
    for e in range(ref.shape[0]):
        scale = np.max(np.abs(ref[e]))
        if scale == 0:
            if np.any(got[e] != 0):
                return float("inf")
            continue
        worst = max(worst, float(np.max(np.abs(got[e] - ref[e])) / max(scale, floor)))
    return worst


LORA_GRADS = ("da_gu", "db_gu", "da_dn", "db_dn")


def compare_layer(got: dict, fw: dict, bw: dict, rgr: dict) -> dict:
    """Errors of every output against the oracle: whole-tensor norm for Y, dX
    and the router gradients, per-expert norm for the LoRA gradients.  Every
    element must be finite (outputs are pre-filled with NaN)."""
    ref = {"y": fw["y"], "dx": bw["dx"], "da_gu": bw["da_gu"], "db_gu": bw["db_gu"],
           "da_dn": bw["da_dn"], "db_dn": bw["db_dn"]}
    if rgr is not None:
        ref["d_topk_w"] = rgr["d_topk_w"]
        ref["d_logits"] = rgr["d_logits"]
    errs = {}
    for key, r in ref.items():
        a = to_numpy_f64(got[key])
        assert a.shape == r.shape, (key, a.shape, r.shape)
        assert np.all(np.isfinite(a)), f"{key}: unwritten or non-finite elements"
        errs[key] = relerr_per_expert(a, r) if key in LORA_GRADS else relerr(a, r)
    return errs
