"""Build the gfx950 HIP library ``libmoe_lora.so`` in-tree with hipcc.

Usage: ``python -m mixture_experts_lora_amd.build`` (or ``build()`` from Python).
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_lora.so")
SOURCES = ("api.hip", "route.hip", "route_noalloc.hip", "gemm.hip", "prepass.hip",
           "grads.hip", "combine.hip", "merge.hip", "layer.hip", "tune.hip", "timing.hip")
# compiled a second time with fp16 elements (-DMOE_F16, objects *_f16.o)
ELEMENT_SOURCES = ("gemm.hip", "prepass.hip", "grads.hip", "combine.hip", "merge.hip")
# the streamed grouped GEMM, once per tile height x stage depth (namespace,
# rows, k per stage), each with bf16 and with fp16 elements
STREAM_TILES = (("t320k64", 320, 64), ("t256k64", 256, 64), ("t320k32", 320, 32), ("t256k32", 256, 32))
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the MoE-LoRA library needs ROCm's hipcc")


def _compile(src: str, extra: list[str], suffix: str = "") -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    warn = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if warn.strip():
        sys.stderr.write(warn + "\n")
    return obj


def build(extra_flags: list[str] | None = None, verbose: bool = True, out: str = LIB,
          objdir: str = OBJ) -> str:
    """Compile every HIP source for gfx950 and link ``libmoe_lora.so``."""
    extra = list(extra_flags or [])
    global OBJ
    OBJ = objdir
    os.makedirs(OBJ, exist_ok=True)
    jobs = [(s, extra, "") for s in SOURCES] + [(s, extra + ["-DMOE_F16"], "_f16") for s in ELEMENT_SOURCES]
    for ns, bm, sk in STREAM_TILES:
        tile = [f"-DMOE_STILE={ns}", f"-DMOE_SBM={bm}", f"-DMOE_SK={sk}"]
        jobs += [("stream.hip", extra + tile, f"_{ns}"), ("stream.hip", extra + tile + ["-DMOE_F16"], f"_{ns}_f16")]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 16)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(sys.argv[1:])
