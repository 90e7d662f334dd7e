"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, answers size queries and rejects bad arguments on the host
before anything is enqueued."""
import ctypes
import os
import re

import pytest

from mixture_experts_lora_amd import _lib
from synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_lora.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmoe_lora.so not built (python -m mixture_experts_lora_amd.build)")
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in ((0, "MOE_SUCCESS"), (1, "MOE_ERROR_INVALID_VALUE"), (2, "MOE_ERROR_UNSUPPORTED"),
                       (3, "MOE_ERROR_WORKSPACE"), (4, "MOE_ERROR_LAUNCH")):
        assert lib.moe_status_string(code).decode() == name


def _dims(**kw):
    base = dict(T=256, d=128, n=64, E=8, k=2, r=4, n_shared=0, lora_scale=1.0)
    base.update(kw)
    return _lib.MoeDims(**base)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_size_queries(lib, name):
    c = CONFIGS[name]
    dm = _dims(T=c.T, d=c.d, n=c.n, E=c.E, k=c.k, r=c.r, n_shared=c.n_shared)
    rs = (c.r + 7) // 8 * 8
    saved = lib.moe_forward_saved_bytes(ctypes.byref(dm))
    assert saved >= c.P_tot * (2 * c.n + c.n + 2 * rs) * 2
    ws = lib.moe_workspace_bytes(ctypes.byref(dm))
    assert ws >= c.P_tot * (c.d + 2 * c.n + 2 * rs) * 2
    assert lib.moe_route_workspace_bytes(ctypes.byref(dm)) >= c.P * 4


BAD = [
    (dict(k=0), 1), (dict(k=9), 1), (dict(T=0), 1), (dict(r=0), 1), (dict(n_shared=2), 1),
    (dict(lora_scale=float("inf")), 1), (dict(lora_scale=float("nan")), 1),
    (dict(d=96), 2), (dict(n=100), 2), (dict(E=300, k=2), 2), (dict(r=129), 2),
    (dict(T=1 << 29, k=8), 2), (dict(dtype=2), 1), (dict(dtype=-1), 1),
    # per-row buffers of 2 GiB or more are outside the 32-bit buffer offsets:
    # O [P_tot, d] = 32768*8 rows x 4096 x 2 B = 2 GiB exactly
    (dict(T=32768, d=4096, n=64, E=8, k=8), 2),
    # G [P_tot, 2n] = 262144 x 8192 x 2 B = 4 GiB
    (dict(T=32768, d=128, n=4096, E=8, k=8), 2),
    # O = 8 GiB
    (dict(T=65536, d=8192, n=64, E=8, k=8), 2),
    # the shared expert's rows count too: (8192*8 + 8192) x 16384 x 2 B = 2.25 GiB
    (dict(T=8192, d=16384, n=64, E=8, k=8, n_shared=1), 2),
]


def test_envelope_just_inside_is_accepted(lib):
    # [P_tot, d] one row short of 2 GiB: 262143 rows would be needed; use
    # P_tot = 32767*8 rows of d = 4096 -> 2 GiB - 64 KiB
    dm = _dims(T=32767, d=4096, n=64, E=8, k=8)
    assert lib.moe_workspace_bytes(ctypes.byref(dm)) > 0
    dm = _dims(T=32768, d=2048, n=2048, E=8, k=8)  # G = 262144 x 4096 x 2 B = 2 GiB
    assert lib.moe_workspace_bytes(ctypes.byref(dm)) == 0
    dm = _dims(T=32768, d=2048, n=2047 // 64 * 64, E=8, k=8)
    assert lib.moe_workspace_bytes(ctypes.byref(dm)) > 0


@pytest.mark.parametrize("kw,code", BAD)
def test_invalid_dims_rejected_on_host(lib, kw, code):
    dm = _dims(**kw)
    assert lib.moe_workspace_bytes(ctypes.byref(dm)) == 0
    assert lib.moe_forward_saved_bytes(ctypes.byref(dm)) == 0
    fake = ctypes.c_void_p(4096)  # never dereferenced: validation fails first
    rt = _lib.MoeRouting(*([4096] * 8))
    assert lib.moe_route(ctypes.byref(dm), fake, ctypes.byref(rt), fake, 1 << 40, None) == code
    w = _lib.MoeWeights(*([4096] * 6))
    assert lib.moe_lora_forward(ctypes.byref(dm), fake, ctypes.byref(rt), ctypes.byref(w), fake,
                                fake, 1 << 40, fake, 1 << 40, None) == code


def test_null_misaligned_and_small_buffers_rejected(lib):
    dm = _dims()
    fake = 4096
    rt = _lib.MoeRouting(*([fake] * 8))
    w = _lib.MoeWeights(*([fake] * 6))
    big = 1 << 40
    # null dims
    assert lib.moe_route(None, fake, ctypes.byref(rt), fake, big, None) == 1
    # null / misaligned pointers
    assert lib.moe_route(ctypes.byref(dm), None, ctypes.byref(rt), fake, big, None) == 1
    assert lib.moe_route(ctypes.byref(dm), fake + 4, ctypes.byref(rt), fake, big, None) == 1
    for i in range(8):  # every routing pointer is required and 16-byte aligned
        ptrs = [fake] * 8
        ptrs[i] = 0
        assert lib.moe_route(ctypes.byref(dm), fake, ctypes.byref(_lib.MoeRouting(*ptrs)), fake, big,
                             None) == 1
        ptrs[i] = fake + 8
        assert lib.moe_route(ctypes.byref(dm), fake, ctypes.byref(_lib.MoeRouting(*ptrs)), fake, big,
                             None) == 1
    bad_w = _lib.MoeWeights(fake, fake, fake + 2, fake, fake, fake)
    assert lib.moe_lora_forward(ctypes.byref(dm), fake, ctypes.byref(rt), ctypes.byref(bad_w), fake,
                                fake, big, fake, big, None) == 1
    # workspace smaller than its query
    need = lib.moe_route_workspace_bytes(ctypes.byref(dm))
    assert lib.moe_route(ctypes.byref(dm), fake, ctypes.byref(rt), fake, need - 1, None) == 3
    saved = lib.moe_forward_saved_bytes(ctypes.byref(dm))
    ws = lib.moe_workspace_bytes(ctypes.byref(dm))
    assert lib.moe_lora_forward(ctypes.byref(dm), fake, ctypes.byref(rt), ctypes.byref(w), fake,
                                fake, saved - 1, fake, ws, None) == 3
    assert lib.moe_lora_forward(ctypes.byref(dm), fake, ctypes.byref(rt), ctypes.byref(w), fake,
                                fake, saved, fake, ws - 1, None) == 3
    assert lib.moe_lora_backward(ctypes.byref(dm), fake, fake, ctypes.byref(rt), ctypes.byref(w),
                                 fake, saved, fake, fake, fake, fake, fake, None, None, fake, ws - 1,
                                 None) == 3
    assert lib.moe_lora_backward(ctypes.byref(dm), fake, fake, ctypes.byref(rt), ctypes.byref(w),
                                 fake, saved, fake, fake, 0, fake, fake, None, None, fake, ws,
                                 None) == 1
    # the optional router-gradient outputs must be aligned when given
    assert lib.moe_lora_backward(ctypes.byref(dm), fake, fake, ctypes.byref(rt), ctypes.byref(w),
                                 fake, saved, fake, fake, fake, fake, fake, fake + 4, None, fake, ws,
                                 None) == 1


def test_python_binding_refuses_cpu_tensors():
    import torch
    import mixture_experts_lora_amd as mel
    dims = mel.Dims(T=4, d=64, n=64, E=2, k=1, r=4)
    with pytest.raises(ValueError):
        mel.route(torch.zeros(4, 2), dims)
    # the autograd wrapper goes through the same checks
    w = mel.Weights(*(torch.zeros(s, dtype=torch.bfloat16) for s in
                      ((2, 128, 64), (2, 64, 64), (2, 64, 4), (2, 4, 128), (2, 64, 4), (2, 4, 64))))
    with pytest.raises(ValueError):
        mel.moe_lora(torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(4, 2), w, dims)


def test_dims_struct_layout():
    # int64 T; six int32; float lora_scale; int32 dtype -> 40 bytes, 8-aligned
    assert ctypes.sizeof(_lib.MoeDims) == 40 and ctypes.alignment(_lib.MoeDims) == 8
    assert _lib.MoeDims.lora_scale.offset == 32 and _lib.MoeDims.dtype.offset == 36


def test_fp16_dims_accepted_and_keyed_apart(lib):
    bf, hf = _dims(d=256), _dims(d=256, dtype=_lib.MOE_F16)
    assert lib.moe_workspace_bytes(ctypes.byref(hf)) == lib.moe_workspace_bytes(ctypes.byref(bf)) > 0
    before = lib.moe_get_engines(ctypes.byref(bf))
    other = before ^ 1
    assert lib.moe_set_engines(ctypes.byref(hf), other) == 0
    assert lib.moe_get_engines(ctypes.byref(hf)) == other
    assert lib.moe_get_engines(ctypes.byref(bf)) == before       # the element type is in the key
    assert lib.moe_set_engines(ctypes.byref(hf), before) == 0


def test_engine_table_on_the_host(lib):
    dm = _lib.MoeDims(T=64, d=128, n=64, E=8, k=2, r=4, n_shared=0, lora_scale=1.0)
    default = lib.moe_get_engines(ctypes.byref(dm))
    assert default == 31                                             # streamed, default tiles
    assert lib.moe_set_engines(ctypes.byref(dm), 1 << 15) == 1      # unknown bit
    assert lib.moe_set_engines(ctypes.byref(dm), 3 << 13) == 1      # split-K field 3 is not a value
    tiles = 31 | (1 << 5) | (1 << 10) | (2 << 13)                    # 256-row gate_up, 32-k down, 4096 chunks
    assert lib.moe_set_engines(ctypes.byref(dm), tiles) == 0
    assert lib.moe_get_engines(ctypes.byref(dm)) == tiles
    assert lib.moe_set_engines(ctypes.byref(dm), 5) == 0
    assert lib.moe_get_engines(ctypes.byref(dm)) == 5
    other = _lib.MoeDims(T=64, d=128, n=64, E=8, k=2, r=8, n_shared=0, lora_scale=1.0)
    assert lib.moe_get_engines(ctypes.byref(other)) == default      # another shape
    dm.T = 999                                                       # T is not part of the key
    assert lib.moe_get_engines(ctypes.byref(dm)) == 5
    assert lib.moe_set_engines(ctypes.byref(dm), default) == 0
    # autotune validates on the host before touching the GPU
    need = lib.moe_autotune_scratch_bytes(ctypes.byref(dm))
    assert need > lib.moe_workspace_bytes(ctypes.byref(dm))
    w = _lib.MoeWeights(*([256] * 6))
    out = ctypes.c_uint(0)
    assert lib.moe_autotune(ctypes.byref(dm), 256, 256, 256, ctypes.byref(w), 256, need - 1, None,
                            ctypes.byref(out)) == 3
    assert lib.moe_autotune(ctypes.byref(dm), 256, 256, 256, ctypes.byref(w), 128, need, None,
                            ctypes.byref(out)) == 1


def test_merged_path_validates_on_the_host(lib):
    dm = _dims()
    fake = 4096
    w = _lib.MoeWeights(*([fake] * 6))
    rt = _lib.MoeRouting(*([fake] * 8))
    assert lib.moe_merge_lora(None, ctypes.byref(w), fake, fake, None) == 1
    assert lib.moe_merge_lora(ctypes.byref(dm), ctypes.byref(w), fake + 2, fake, None) == 1
    assert lib.moe_merge_lora(ctypes.byref(dm), ctypes.byref(w), fake, None, None) == 1
    bad_w = _lib.MoeWeights(fake, fake, fake, fake + 8, fake, fake)
    assert lib.moe_merge_lora(ctypes.byref(dm), ctypes.byref(bad_w), fake, fake, None) == 1
    dbad = _dims(d=96)
    assert lib.moe_merge_lora(ctypes.byref(dbad), ctypes.byref(w), fake, fake, None) == 2
    saved = lib.moe_forward_saved_bytes(ctypes.byref(dm))
    ws = lib.moe_workspace_bytes(ctypes.byref(dm))
    assert lib.moe_forward_merged(ctypes.byref(dm), fake, ctypes.byref(rt), fake, fake, fake, fake,
                                  saved, fake, ws - 1, None) == 3
    assert lib.moe_forward_merged(ctypes.byref(dm), fake, ctypes.byref(rt), fake, fake + 4, fake, fake,
                                  saved, fake, ws, None) == 1
    assert lib.moe_forward_merged(ctypes.byref(dbad), fake, ctypes.byref(rt), fake, fake, fake, fake,
                                  saved, fake, ws, None) == 2
