#!/usr/bin/env python3
"""Benchmark: MoE-LoRA layer fwd+bwd tokens/s on one MI355X.

One step = route + forward + backward of the Qwen3-30B-A3B-shaped layer
(T=4096, d=2048, n=768, E=128, top-8, LoRA rank 64 on gate_up and down, bf16,
router logits N(0,1)) on seeded synthetic inputs already resident in HBM.

Prints ONE JSON line.  Besides the standard benchmark fields it carries
  roofline      the dominant kernel (the gate_up grouped GEMM) against its
                bound, from HIP-event timing of every launch over a second
                timed region of the same steps;
  step_roofline the whole step against max(FLOPs / MFMA peak, minimum
                bytes / HBM peak);
  gemm_mfma_frac  algorithmic grouped-GEMM FLOPs / summed GEMM kernel time /
                bf16 dense MFMA peak;
  kernels_us    average duration per kernel;
  router_grads  the optional routing-weight / logit gradients (the pages freeze
                the router, so they are not part of the step): a third timed
                region of backward calls that also produce them, its extra
                time per step and the router_grad kernel against HBM peak;
  engines       the engine and tile configuration of each product (the
                one-time autotune's choice, made before the warm-up steps,
                unless --no-autotune);
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload;
  cpu_naive_loop  the oracle's per-expert search loop (the pages' starting
                point), forward only, float64, timed the same way, as context;
  configs       the other workloads (tiny, deepseek_shared, long_zipf,
                routing_stress, and the headline shape with fp16 elements),
                each autotuned and timed for ms/step, tokens/s, TFLOP/s, step
                roofline fraction and grouped-GEMM fraction of the bf16 peak,
                next to its time under the build's default engines.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-LoRA layer fwd+bwd tokens/s; grouped-GEMM % of bf16 MFMA peak"
PEAK_BF16 = 2516.6e12   # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s
# grouped products; the four LoRA gradients run as one launch ("lora_grads")
# at ranks <= 64, as four above
GEMM_KERNELS = ("gate_up", "down", "dh", "dx", "prepass_xa", "prepass_ha", "prepass_qdn",
                "prepass_qgu", "lora_grads", "grad_db_dn", "grad_da_dn", "grad_db_gu", "grad_da_gu")
# per-kernel algorithmic work is per launch; the timer reports per-launch averages


def kernel_work(c):
    """Algorithmic FLOPs and unique HBM bytes of one launch of each kernel.

    Bytes count every input read once and every output written once (bf16 =
    2 B, fp32 = 4 B); re-reads of gathered rows are cache traffic, not
    algorithmic bytes."""
    T, d, n, r, k, S = c.T, c.d, c.n, c.r, c.k, c.n_shared
    P = T * k + S * T
    Et = c.E + S
    b = 2
    W_gu, W_dn = Et * 2 * n * d * b, Et * d * n * b
    A_gu, B_gu, A_dn, B_dn = Et * d * r * b, Et * r * 2 * n * b, Et * n * r * b, Et * r * d * b
    X = T * d * b
    G, H, R, O = P * 2 * n * b, P * n * b, P * r * b, P * d * b
    idx = P * 4 * 2
    logits = c.T * c.E * 4
    # ids and weights, counts, offsets, the permutation and its inverse, and
    # the gather table (token and weight of every sorted row)
    route_out = c.T * c.k * 4 * 2 + c.E * 4 + (c.E + 1) * 4 + c.T * c.k * 4 * 2 + P * 4 * 2
    work = {
        "route": (0, logits + route_out),
        "prepass_xa": (2 * P * d * r, X + A_gu + R + idx),
        "gate_up": (2 * P * d * 2 * n + 2 * P * r * 2 * n, W_gu + B_gu + X + R + G + H + idx),
        "prepass_ha": (2 * P * n * r, H + A_dn + R),
        "down": (2 * P * n * d + 2 * P * r * d, W_dn + B_dn + H + R + O),
        "combine_y": (2 * P * d, O + T * d * b + idx),
        "prepass_qdn": (2 * P * d * r, X + B_dn + R + idx),
        "dh": (2 * P * d * n + 2 * P * r * n, W_dn + A_dn + X + R + 2 * G + idx),
        "prepass_qgu": (2 * P * 2 * n * r, G + B_gu + R),
        "dx": (2 * P * 2 * n * d + 2 * P * r * d, W_gu + A_gu + G + R + O),
        "combine_dx": (P * d, O + T * d * b + idx),
        "grad_db_dn": (2 * P * r * d, R + X + Et * r * d * 4 + idx),
        "grad_da_dn": (2 * P * n * r, H + R + Et * n * r * 4),
        "grad_db_gu": (2 * P * r * 2 * n, R + G + Et * r * 2 * n * 4),
        "grad_da_gu": (2 * P * d * r, X + R + Et * d * r * 4 + idx),
        # partials per 64-column group, pair positions, weights and ids in;
        # d_topk_w and d_logits out
        "router_grad": (0, T * k * (n // 64) * 4 + 3 * T * k * 4 + T * k * 4 + T * c.E * 4),
    }
    four = [work[g] for g in ("grad_db_dn", "grad_da_dn", "grad_db_gu", "grad_da_gu")]
    work["lora_grads"] = (sum(f for f, _ in four), sum(b for _, b in four))
    return work


def step_roofline(c, ms):
    """The whole step (route + forward + backward) against its roofline:
    t_roof = max(algorithmic FLOPs / bf16 peak, minimum bytes / HBM peak).

    FLOPs: forward 6 P d n + 2 P r (2d + 3n), backward 6 P d n + 4 P r (2d + 3n)
    (no base-weight gradient; each X A / H A product once).  Minimum bytes:
    logits once, X twice, dY once, W_gu and W_dn twice, the LoRA factors
    twice, G and the rank-r saves written and read, Y and dX written, the
    fp32 LoRA gradients written."""
    T, d, n, r, k, S, E = c.T, c.d, c.n, c.r, c.k, c.n_shared, c.E
    P, Et, b = T * k + S * T, E + S, 2
    flops = (6 * P * d * n + 2 * P * r * (2 * d + 3 * n)) + (6 * P * d * n + 4 * P * r * (2 * d + 3 * n))
    lora = Et * r * (d + 2 * n + n + d)
    byts = (T * E * 4 + 3 * T * d * b + 2 * Et * 3 * n * d * b + 2 * lora * b
            + 2 * P * 2 * n * b + 2 * 2 * P * r * b + 2 * T * d * b + lora * 4)
    t_f, t_b = flops / PEAK_BF16, byts / PEAK_HBM
    t_roof = max(t_f, t_b)
    return {"bound": "hbm" if t_b >= t_f else "mfma", "t_roof_us": round(t_roof * 1e6, 1),
            "t_us": round(ms * 1e3, 1), "frac": t_roof / (ms * 1e-3),
            "algorithmic_flops": flops, "min_bytes": byts}


def cpu_baseline(dims, inp, budget_s: float):
    """The oracle (float32, numpy) timed on the host cores: route + forward +
    backward on the first T_s tokens of the same inputs (T_s grows until one
    pass takes about budget_s / 3, capped at the whole workload), median of
    three passes; tokens/s = T_s / median wall time."""
    import dataclasses
    import statistics

    import numpy as np
    import oracle

    # BLAS threads: threadpoolctl when it recognises numpy's BLAS, else the
    # variables OpenBLAS reads, else every core
    env_threads = os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get("OMP_NUM_THREADS")
    threads = int(env_threads) if env_threads and env_threads.isdigit() else os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        found = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if found:
            threads = max(found)
    except Exception:  # pragma: no cover
        pass
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:  # pragma: no cover
        blas = "unknown"
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass

    def one(Ts):
        sd = dataclasses.replace(dims, T=Ts)
        sub = dataclasses.replace(inp, dims=sd, logits=inp.logits[:Ts], x=inp.x[:Ts], dy=inp.dy[:Ts])
        t0 = time.perf_counter()
        ids, w = oracle.topk_softmax(sub.logits, sd.k)
        oracle.route(ids, sd.E)
        oracle.forward(sub, ids, w, sd, dtype=np.float32)
        oracle.backward(sub, ids, w, sd, dtype=np.float32)
        return time.perf_counter() - t0

    Ts = 64
    dt = one(Ts)
    while dt < budget_s / 3 and Ts < dims.T:
        Ts = min(dims.T, max(Ts * 2, int(Ts * budget_s / 3 / max(dt, 1e-3))))
        dt = one(Ts)
    med = statistics.median([dt, one(Ts), one(Ts)])
    return {"value": Ts / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {Ts} of {dims.T} tokens (same seeded inputs), float32 numpy "
                      f"route+forward+backward, median of 3 passes = {med:.2f} s",
            "blas": blas, "host_cpu": cpu, "host_cpus": os.cpu_count()}


CROSSOVER_T = (1024, 2048, 4096, 8192, 12288, 16384, 24576, 32768, 49152)


def crossover(args):
    """Split LoRA against the merged-weight path the pages compare it with
    (faster-MoE page, "MoE LoRA changes things"), forward only, at the
    Qwen3-30B-A3B shapes (d 2048, n 768, E 128, top-8, r 64) for a range of
    token counts T: the split forward (rank-r pre-passes, grouped products
    with their low-rank pass, combine) against merging W + s (A B)^T for
    every expert and running the grouped products on the merged weights.
    The inputs are the first T tokens of one seeded draw; the weights are
    the same for every T.  Prints one JSON line with the times and the
    crossover T (linear interpolation where merged first beats split) next
    to the page's FLOP-count formulas."""
    import numpy as np
    import torch

    import mixture_experts_lora_amd as mel
    from synth import CONFIGS, make_inputs

    base = CONFIGS["qwen3_30b_a3b"]
    big = dataclasses.replace(base, T=max(CROSSOVER_T))
    inp = make_inputs(big, seed=0)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    w = mel.Weights(bf(inp.w_gu), bf(inp.w_dn), bf(inp.a_gu), bf(inp.b_gu), bf(inp.a_dn), bf(inp.b_dn))
    X, L = bf(inp.x), torch.from_numpy(inp.logits).cuda()
    merged = mel.MergedWeights(torch.empty_like(w.w_gate_up), torch.empty_like(w.w_down))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    rows = []
    for T in CROSSOVER_T:
        c = dataclasses.replace(base, T=T)
        dims = mel.Dims(c.T, c.d, c.n, c.E, c.k, c.r, c.n_shared, c.lora_scale)
        layer = mel.MoELoRALayer(dims, w)
        x = X[:T].contiguous()
        layer.route(L[:T].contiguous())
        y_m = torch.empty_like(x)
        reps = 10 if T <= 16384 else 5
        split = timed(lambda: layer.forward(x), reps)
        merge = timed(lambda: mel.merge_lora(w, dims, out=merged), reps)
        fwd_m = timed(lambda: mel.forward_merged(x, layer.routing, merged, dims, y=y_m, saved=layer.saved,
                                                 ws=layer.ws), reps)
        both = timed(lambda: (mel.merge_lora(w, dims, out=merged),
                              mel.forward_merged(x, layer.routing, merged, dims, y=y_m, saved=layer.saved,
                                                 ws=layer.ws)), reps)
        rows.append({"T": T, "split_ms": round(split, 4), "merged_ms": round(both, 4),
                     "merge_only_ms": round(merge, 4), "merged_products_ms": round(fwd_m, 4)})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        del layer
        torch.cuda.empty_cache()
    cross = None
    for a, b in zip(rows, rows[1:]):
        da, db = a["merged_ms"] - a["split_ms"], b["merged_ms"] - b["split_ms"]
        if da > 0 >= db:
            cross = round(a["T"] + (b["T"] - a["T"]) * da / (da - db))
            break
    E, m, n, k, r = base.E, base.d, base.n, base.k, base.r
    out = {"metric": "split vs merged LoRA forward, ms", "config": {
        "workload": "qwen3_30b_a3b shapes, forward only", "d": m, "n": n, "E": E, "top_k": k,
        "lora_rank": r, "dtype": "bf16"},
        "rows": rows, "measured_crossover_T": cross,
        "page_formula_T": {"per projection (m, n) = (2048, 768)": round(E * m * n / (k * (m + n)) * (1 + 1 / (2 * r))),
                           "fused gate_up (m, 2n)": round(E * m * 2 * n / (k * (m + 2 * n)) * (1 + 1 / (2 * r))),
                           "whole layer (gate_up + down)": round(E * (2 * r + 1) * (m * 2 * n + n * m)
                                                                 / (2 * k * r * ((m + 2 * n) + (n + m))))}}
    print(json.dumps(out), flush=True)


# the workloads besides the headline one, each measured in the same run
OTHER_CONFIGS = (("tiny", "bf16"), ("deepseek_shared", "bf16"), ("long_zipf", "bf16"),
                 ("routing_stress", "bf16"), ("qwen3_30b_a3b", "f16"))


def measure_config(name: str, dtype: str, steps: int, warmup: int) -> dict:
    """One workload: the one-time autotune, then route + forward + backward
    steps under the build's default engines and under the autotuned ones
    (HIP events around each timed region), and one event-timed pass of the
    autotuned steps for the per-kernel figures."""
    import numpy as np
    import torch

    import mixture_experts_lora_amd as mel
    from mixture_experts_lora_amd import _lib
    from synth import CONFIGS, make_inputs

    c = dataclasses.replace(CONFIGS[name], element=dtype)
    inp = make_inputs(c, seed=0)
    dims = mel.Dims(c.T, c.d, c.n, c.E, c.k, c.r, c.n_shared, c.lora_scale,
                    mel.MOE_F16 if dtype == "f16" else mel.MOE_BF16)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(dims.elem)

    w = mel.Weights(up(inp.w_gu), up(inp.w_dn), up(inp.a_gu), up(inp.b_gu), up(inp.a_dn), up(inp.b_dn))
    logits = torch.from_numpy(inp.logits).cuda()
    x, dy = up(inp.x), up(inp.dy)
    layer = mel.MoELoRALayer(dims, w)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def step():
        layer.route(logits)
        layer.forward(x)
        layer.backward(dy, x)

    def timed():
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    chosen = mel.autotune(dims, logits, x, dy, w)
    mel.set_engines(dims, mel.ENGINE_ALL)
    default_ms = timed()
    mel.set_engines(dims, chosen)
    ms = timed()
    _lib.timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    rep = _lib.timing_report()
    _lib.timing_enable(False)
    work = kernel_work(c)
    gemm_flops = sum(work[k][0] for k in GEMM_KERNELS if k in rep)
    gemm_time = sum(rep[k][0] for k in GEMM_KERNELS if k in rep) / steps * 1e-3
    gu_us = 1e3 * rep["gate_up"][0] / rep["gate_up"][1]
    avg_us = {k: 1e3 * v[0] / v[1] for k, v in rep.items()}
    route_us = sum(avg_us.get(k, 0.0) for k in ("route_select", "route_scatter"))
    mem = {"route": {"us": round(route_us, 2), "GB/s": round(work["route"][1] / route_us / 1e3, 1)}}
    for k in ("combine_y", "combine_dx"):
        mem[k] = {"us": round(avg_us[k], 2), "GB/s": round(work[k][1] / avg_us[k] / 1e3, 1)}
    for v in mem.values():
        v["frac_of_hbm_peak"] = round(v["GB/s"] * 1e9 / PEAK_HBM, 3)
    roof = step_roofline(c, ms)
    out = {"T": c.T, "d": c.d, "n": c.n, "E": c.E, "top_k": c.k, "lora_rank": c.r,
           "n_shared": c.n_shared, "logits": c.logits_recipe, "dtype": dtype,
           "ms_per_step": round(ms, 4), "default_engines_ms_per_step": round(default_ms, 4),
           "tokens_per_s": round(c.T / (ms * 1e-3), 1),
           "tflop_s": round(roof["algorithmic_flops"] / (ms * 1e-3) / 1e12, 1),
           "step_roofline": {k: roof[k] for k in ("bound", "t_roof_us", "frac")},
           "gemm_mfma_frac": round(gemm_flops / gemm_time / PEAK_BF16, 4),
           "gemm_tflops": round(gemm_flops / gemm_time / 1e12, 1),
           "gate_up": {"us": round(gu_us, 2), "tflop_s": round(work["gate_up"][0] / gu_us / 1e6, 1),
                       "GB/s": round(work["gate_up"][1] / gu_us / 1e3, 1)},
           "memory_bound_kernels": mem,
           "engines": {"bits": chosen, **mel.describe_engines(chosen)}}
    del layer, w, x, dy, logits
    torch.cuda.empty_cache()
    return out


def cpu_naive_loop(dims, inp, budget_s: float):
    """The per-expert search loop the pages start from (oracle.forward_naive:
    every expert finds its tokens with a data-dependent query, runs its MLP on
    them and adds the weighted result), float64 numpy, forward only, on the
    first T_s tokens (T_s grows until one pass takes about budget_s / 3);
    context beside cpu_baseline, not a target."""
    import statistics

    import numpy as np
    import oracle

    def one(Ts):
        sd = dataclasses.replace(dims, T=Ts)
        sub = dataclasses.replace(inp, dims=sd, logits=inp.logits[:Ts], x=inp.x[:Ts], dy=inp.dy[:Ts])
        t0 = time.perf_counter()
        ids, w = oracle.topk_softmax(sub.logits, sd.k)
        oracle.forward_naive(sub, ids, w, sd, dtype=np.float64)
        return time.perf_counter() - t0

    Ts = 64
    dt = one(Ts)
    while dt < budget_s / 3 and Ts < dims.T:
        Ts = min(dims.T, max(Ts * 2, int(Ts * budget_s / 3 / max(dt, 1e-3))))
        dt = one(Ts)
    med = statistics.median([dt, one(Ts), one(Ts)])
    return {"value": Ts / med, "unit": "tokens/s (forward only)", "kind": "oracle per-expert loop, float64",
            "sample": f"first {Ts} of {dims.T} tokens, route + forward, median of 3 passes = {med:.2f} s"}


def measured_traffic(kernel: str, workload: str, tile: str):
    """HBM bytes per launch of `kernel` in tile configuration `tile` (e.g.
    t320k64) from the committed rocprofv3 counter summary, or None when that
    configuration was not measured or the kernel source changed since."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch\[" + tile + r"\]:\s*([0-9]+)", text)
    m_src = re.search(r"source_files:\s*(.+)", text)
    if not (m_sha and m_b and m_src):
        return None
    h = hashlib.sha256()
    for name in m_src.group(1).split():
        h.update(open(os.path.join(ROOT, "mixture_experts_lora_amd", "csrc", name), "rb").read())
    if h.hexdigest() != m_sha.group(1):
        return None
    return int(m_b.group(1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3_30b_a3b")
    ap.add_argument("--dtype", choices=("bf16", "f16"), default="bf16",
                    help="16-bit element type of activations and weights")
    ap.add_argument("--no-autotune", action="store_true",
                    help="keep the build's default engines instead of the one-time autotune")
    ap.add_argument("--engines", type=int, default=None, metavar="BITS",
                    help="use this engine/tile word instead of the autotune (for profiling)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of CPU oracle work for cpu_baseline (0 = skip)")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only the headline workload (skip the `configs` object)")
    ap.add_argument("--crossover", action="store_true",
                    help="time split LoRA against merged weights over a range of T and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device (known-size kernel for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch

        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.int32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 3}))
        return
    if args.crossover:
        crossover(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this layer's data-parallel shards are independent and are not run here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_lora_amd as mel
    from mixture_experts_lora_amd import _lib
    from synth import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mel.load()
    c = dataclasses.replace(CONFIGS[args.config], element=args.dtype)
    inp = make_inputs(c, seed=0)
    dims = mel.Dims(c.T, c.d, c.n, c.E, c.k, c.r, c.n_shared, c.lora_scale,
                    mel.MOE_F16 if args.dtype == "f16" else mel.MOE_BF16)

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(dims.elem)

    w = mel.Weights(bf(inp.w_gu), bf(inp.w_dn), bf(inp.a_gu), bf(inp.b_gu), bf(inp.a_dn),
                    bf(inp.b_dn))
    logits = torch.from_numpy(inp.logits).cuda()
    x, dy = bf(inp.x), bf(inp.dy)
    layer = mel.MoELoRALayer(dims, w)
    # one-time per-shape engine autotune before any timed step (untimed, as
    # the start-up autotune of the pages' kernels)
    if args.engines is not None:
        mel.set_engines(dims, args.engines)
        engines = args.engines
    else:
        engines = mel.get_engines(dims) if args.no_autotune else mel.autotune(dims, logits, x, dy, w)

    def step():
        layer.route(logits)
        layer.forward(x)
        layer.backward(dy, x)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps

    # the same step timed one at a time (each between its own pair of events),
    # 50 of them after 10 more warm-ups: the distribution behind the mean
    for _ in range(10):
        step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    single = sorted(a.elapsed_time(b) for a, b in ev)
    single_step = {"n": len(single), "median_ms": round(single[len(single) // 2], 4),
                "p10_ms": round(single[len(single) // 10], 4),
                "p90_ms": round(single[(9 * len(single)) // 10], 4)}

    # second timed region: the same steps with every kernel bracketed by events
    _lib.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    rep = _lib.timing_report()
    _lib.timing_enable(False)
    per_step = args.steps
    work = kernel_work(c)
    avg_us = {k: 1e3 * v[0] / v[1] for k, v in rep.items()}
    gemm_flops = sum(work[k][0] for k in GEMM_KERNELS if k in rep)
    gemm_time = sum(rep[k][0] for k in GEMM_KERNELS if k in rep) / per_step * 1e-3
    dom = "gate_up"
    f, byts = work[dom]
    t_dom = avg_us[dom] * 1e-6
    hbm_bound = byts / PEAK_HBM >= f / PEAK_BF16
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": byts / t_dom / 1e9, "peak": PEAK_HBM / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": f / t_dom / 1e12, "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    gu_tile = f"t{256 if engines & mel.TILE256(0) else 320}k{32 if engines & mel.STAGE32(0) else 64}"
    roof["traffic"] = (measured_traffic(dom, args.config if args.dtype == "bf16"
                                        else f"{args.config}_{args.dtype}", gu_tile)
                       if engines & mel.ENGINE_GATE_UP else None)
    roof["tile"] = gu_tile
    roof["kernel"] = dom
    roof["kernel_us"] = avg_us[dom]
    roof["algorithmic_bytes"] = byts
    roof["algorithmic_flops"] = f
    roof["mfma_frac"] = f / t_dom / PEAK_BF16

    # routing (all its launches) and the two combines against the HBM peak
    mem = {}
    route_us = sum(avg_us.get(k, 0.0) for k in ("route_select", "route_scatter"))
    if route_us > 0:
        mem["route"] = {"us": round(route_us, 2), "GB/s": round(work["route"][1] / route_us / 1e3, 1)}
    for k in ("combine_y", "combine_dx"):
        if k in avg_us:
            mem[k] = {"us": round(avg_us[k], 2), "GB/s": round(work[k][1] / avg_us[k] / 1e3, 1)}
    for v in mem.values():
        v["frac_of_hbm_peak"] = round(v["GB/s"] * 1e9 / PEAK_HBM, 3)

    # the same step captured once as a HIP graph and replayed: the kernels and
    # their work are unchanged, the host launch gaps between them are gone
    def graph_ms():
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        del g
        return t0.elapsed_time(t1) / args.steps

    g_ms = graph_ms()
    graph = {"ms_per_step": round(g_ms, 4), "tokens_per_s": round(c.T / (g_ms * 1e-3), 1)}

    # optional router gradients: backward alone, without and with them
    def bwd_ms(router):
        for _ in range(2):
            layer.backward(dy, x, router=router)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(args.steps):
            layer.backward(dy, x, router=router)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    b_plain, b_router = bwd_ms(False), bwd_ms(True)
    _lib.timing_enable(True)
    for _ in range(args.steps):
        layer.backward(dy, x, router=True)
    torch.cuda.synchronize()
    rrep = _lib.timing_report()
    _lib.timing_enable(False)
    rg_us = 1e3 * rrep["router_grad"][0] / rrep["router_grad"][1]
    rg_bytes = work["router_grad"][1]
    router = {"backward_ms": round(b_plain, 4), "backward_with_router_ms": round(b_router, 4),
              "router_grad_us": round(rg_us, 2), "router_grad_GB/s": round(rg_bytes / rg_us / 1e3, 1),
              "router_grad_frac_of_hbm_peak": round(rg_bytes / (rg_us * 1e-6) / PEAK_HBM, 3),
              "algorithmic_bytes": rg_bytes}

    out = {
        "metric": METRIC,
        "value": c.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "single_step_ms": single_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded normal draws; no dataset, random-init weights)",
        "config": {"workload": f"{c.name}: MoE-LoRA expert layer route+fwd+bwd", "T": c.T,
                   "d": c.d, "n": c.n, "E": c.E, "top_k": c.k, "lora_rank": c.r,
                   "n_shared": c.n_shared, "logits": c.logits_recipe},
        "gemm_mfma_frac": gemm_flops / gemm_time / PEAK_BF16,
        "gemm_tflops": gemm_flops / gemm_time / 1e12,
        "roofline": roof,
        "step_roofline": step_roofline(c, ms),
        "kernels_us": {k: round(v, 2) for k, v in sorted(avg_us.items())},
        "memory_bound_kernels": mem,
        "graph_replay": graph,
        "router_grads": router,
        "engines": {"bits": engines, "autotuned": not args.no_autotune and args.engines is None,
                    **mel.describe_engines(engines)},
    }
    if args.cpu_budget > 0:
        out["cpu_baseline"] = cpu_baseline(c, inp, args.cpu_budget)
        out["cpu_naive_loop"] = cpu_naive_loop(c, inp, min(args.cpu_budget, 6.0))
    if not args.no_configs:
        del layer, w, x, dy, logits
        torch.cuda.empty_cache()
        out["configs"] = {}
        for name, dt in OTHER_CONFIGS:
            if (name, dt) == (args.config, args.dtype):
                continue
            key = name if dt == "bf16" else f"{name}_{dt}"
            out["configs"][key] = measure_config(name, dt, min(args.steps, 10), min(args.warmup, 3))
            print(f"[bench] {key}: {out['configs'][key]['ms_per_step']} ms/step", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
