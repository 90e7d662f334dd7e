"""ctypes view of the C ABI in include/moe_lora.h (loading and signatures only)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_lora.so")

MOE_SUCCESS = 0
MOE_ERROR_INVALID_VALUE = 1
MOE_ERROR_UNSUPPORTED = 2
MOE_ERROR_WORKSPACE = 3
MOE_ERROR_LAUNCH = 4

MOE_BF16 = 0
MOE_F16 = 1

MOE_ROUTE_NOALLOC_SCRATCH_BYTES = 4 << 20

EXPORTED = (
    "moe_status_string",
    "moe_route_workspace_bytes",
    "moe_forward_saved_bytes",
    "moe_workspace_bytes",
    "moe_route",
    "moe_route_noalloc",
    "moe_lora_forward",
    "moe_lora_backward",
    "moe_merge_lora",
    "moe_forward_merged",
    "moe_set_engines",
    "moe_get_engines",
    "moe_autotune_scratch_bytes",
    "moe_autotune",
    "moe_timing_enable",
    "moe_timing_report",
)


class MoeDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("n", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("r", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("lora_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class MoeRouting(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("topk_ids", "topk_w", "counts", "offsets", "sorted_pair", "pair_pos",
                 "row_token", "row_weight")]


class MoeWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("w_gate_up", "w_down", "a_gate_up", "b_gate_up", "a_down", "b_down")]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once.  There is no fallback: a missing library is
    an error, the layer only runs through these kernels."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mixture_experts_lora_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pd = ctypes.POINTER(MoeDims)
    pr = ctypes.POINTER(MoeRouting)
    pw = ctypes.POINTER(MoeWeights)
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    for q in ("moe_route_workspace_bytes", "moe_forward_saved_bytes", "moe_workspace_bytes"):
        getattr(lib, q).restype = sz
        getattr(lib, q).argtypes = [pd]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_route.argtypes = [pd, vp, pr, vp, sz, vp]
    lib.moe_route_noalloc.restype = ctypes.c_int
    lib.moe_route_noalloc.argtypes = [pd, vp, pr, vp]
    lib.moe_lora_forward.restype = ctypes.c_int
    lib.moe_lora_forward.argtypes = [pd, vp, pr, pw, vp, vp, sz, vp, sz, vp]
    lib.moe_lora_backward.restype = ctypes.c_int
    lib.moe_lora_backward.argtypes = [pd, vp, vp, pr, pw, vp, sz, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_merge_lora.restype = ctypes.c_int
    lib.moe_merge_lora.argtypes = [pd, pw, vp, vp, vp]
    lib.moe_forward_merged.restype = ctypes.c_int
    lib.moe_forward_merged.argtypes = [pd, vp, pr, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.moe_set_engines.restype = ctypes.c_int
    lib.moe_set_engines.argtypes = [pd, ctypes.c_uint]
    lib.moe_get_engines.restype = ctypes.c_uint
    lib.moe_get_engines.argtypes = [pd]
    lib.moe_autotune_scratch_bytes.restype = sz
    lib.moe_autotune_scratch_bytes.argtypes = [pd]
    lib.moe_autotune.restype = ctypes.c_int
    lib.moe_autotune.argtypes = [pd, vp, vp, vp, pw, vp, sz, vp, ctypes.POINTER(ctypes.c_uint)]
    lib.moe_timing_enable.restype = ctypes.c_int
    lib.moe_timing_enable.argtypes = [ctypes.c_int]
    lib.moe_timing_report.restype = ctypes.c_int
    lib.moe_timing_report.argtypes = [ctypes.c_char_p, ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                                      ctypes.POINTER(ctypes.c_int), ctypes.c_int]
    _lib = lib
    return lib


def timing_enable(on: bool) -> None:
    check(load().moe_timing_enable(1 if on else 0), "moe_timing_enable")


def timing_report(max_entries: int = 64, name_len: int = 64) -> dict:
    """{kernel name: (total ms, launches)} for the kernels recorded since the
    last enable/report."""
    names = ctypes.create_string_buffer(max_entries * name_len)
    ms = (ctypes.c_float * max_entries)()
    cnt = (ctypes.c_int * max_entries)()
    n = load().moe_timing_report(names, name_len, ms, cnt, max_entries)
    if n < 0:
        raise RuntimeError("moe_timing_report: HIP error")
    raw = names.raw
    out = {}
    for i in range(n):
        nm = raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode()
        out[nm] = (float(ms[i]), int(cnt[i]))
    return out


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status != MOE_SUCCESS:
        raise MoeError(status, where)
