"""bench.py's host-side arithmetic, without a GPU: the whole-step roofline
(FLOPs and minimum bytes) against the per-kernel work table it also reports,
and against the per-workload figures worked out from the layer's shapes in
the measurement plan (699.0 GFLOP / 3.14 GB for the Qwen3-30B-A3B-shaped
layer, and so on); and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import CONFIGS  # noqa: E402

# (GFLOP fwd+bwd, minimum GB, roofline us, bound) per workload
PLAN = {
    "qwen3_30b_a3b": (699.0, 3.14, 392, "hbm"),
    "deepseek_shared": (1563.3, 3.17, 621, "mfma"),
    "long_zipf": (6568.3, 5.20, 2610, "mfma"),
    "routing_stress": (5592.0, 5.27, 2222, "mfma"),
}
GEMMS = ("gate_up", "down", "dh", "dx", "prepass_xa", "prepass_ha", "prepass_qdn", "prepass_qgu",
         "grad_db_dn", "grad_da_dn", "grad_db_gu", "grad_da_gu")


@pytest.mark.parametrize("name", list(PLAN))
def test_step_roofline_matches_plan(name):
    gf, gb, us, bound = PLAN[name]
    r = bench.step_roofline(CONFIGS[name], ms=1.0)
    assert abs(r["algorithmic_flops"] / 1e9 - gf) < 0.05
    assert abs(r["min_bytes"] / 1e9 - gb) < 0.005
    assert abs(r["t_roof_us"] - us) < 1.0
    assert r["bound"] == bound


@pytest.mark.parametrize("name", list(CONFIGS))
def test_step_flops_equal_sum_of_kernels(name):
    c = CONFIGS[name]
    work = bench.kernel_work(c)
    assert sum(work[g][0] for g in GEMMS) == bench.step_roofline(c, ms=1.0)["algorithmic_flops"]
    # the one-launch LoRA gradient kernel carries the four gradients' work
    assert work["lora_grads"][0] == sum(work[g][0] for g in GEMMS if g.startswith("grad_"))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_hip_flags_keep_packed_fp32_off():
    """Every HIP object is compiled with the packed-fp32 instructions turned
    off (the compiler would otherwise form them from plain float code)."""
    from mixture_experts_lora_amd import build
    flags = build.HIPCC_FLAGS
    i = flags.index("-packed-fp32-ops")
    assert flags[i - 3:i + 1] == ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    assert "--offload-arch=gfx950" in flags
