"""Benchmark of the MoE expert layer on one MI355X.

One step = one forward and one backward of the whole layer (route, permute,
grouped SwiGLU FFN, combine and the backward of each) on the Qwen3-30B-A3B
shaped workload with the balanced gate: T=4096 tokens, d=2048, E=128 experts,
k=8, I=768, bf16 storage with fp32 accumulation, seeded synthetic inputs that
are resident in HBM before the timed region.

Prints ONE JSON line (rank 0) with tokens/s, the roofline of the dominant
kernel (timed with HIP events on its launch stream during the timed region)
and the CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s fwd+bwd and grouped-GEMM MFMA util @ Qwen3-30B-A3B shape"
WORKLOAD = "qwen3_balanced_fwdbwd_T4096_d2048_E128_k8_I768"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = ["gemm.hip", "gemm.h", "common.h"]

# Algorithmic work per launch of each GEMM kernel: (flops, bytes) as functions
# of R routed rows, d, I, E_loc.  Bytes: every operand read once, every output
# written once, bf16 (2 bytes).
GEMMS = {
    "ffn_gateup_fwd":   (lambda R, d, I, El: 4 * R * d * I,
                         lambda R, d, I, El: 2 * (R * d + 2 * El * d * I + 2 * R * I + R * I)),
    "ffn_down_fwd":     (lambda R, d, I, El: 2 * R * I * d,
                         lambda R, d, I, El: 2 * (R * I + El * I * d + R * d)),
    "ffn_down_dgrad":   (lambda R, d, I, El: 2 * R * d * I,
                         lambda R, d, I, El: 2 * (R * d + El * I * d + 2 * R * I + 2 * R * I)),
    "ffn_gateup_dgrad": (lambda R, d, I, El: 4 * R * d * I,
                         lambda R, d, I, El: 2 * (2 * R * I + 2 * El * d * I + R * d)),
    "ffn_down_wgrad":   (lambda R, d, I, El: 2 * R * I * d,
                         lambda R, d, I, El: 2 * (R * I + R * d + El * I * d)),
    "ffn_gateup_wgrad": (lambda R, d, I, El: 4 * R * d * I,
                         lambda R, d, I, El: 2 * (R * d + 2 * R * I + 2 * El * d * I)),
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_50_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(budget_s: float):
    """The oracle (numpy fp64) timed on the host on a bounded sample of the
    workload: the same layer with the first T_s tokens (balanced gate, so every
    expert keeps an equal share of rows)."""
    import numpy as np
    import moe_inputs as MI
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    w = MI.WORKLOADS[WORKLOAD]
    a = MI.generate(w)

    def step(Ts):
        x, dY = a["x"][:Ts], a["dY"][:Ts]
        t0 = time.perf_counter()
        f = O.layer_fwd(x, a["Wr"], None, a["Wg"], a["Wu"], a["Wd"], w.k, w.gate, w.E)
        O.layer_bwd(f, dY, x, a["Wr"], a["Wg"], a["Wu"], a["Wd"], w.k, w.gate)
        return time.perf_counter() - t0

    t_probe = step(256)
    Ts = int(min(w.T, max(256, 256 * budget_s / max(t_probe, 1e-3))) // 256 * 256)
    dt = step(Ts)
    return {"value": round(Ts / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one fwd+bwd of the layer on the first {Ts} of {w.T} tokens "
                      f"(balanced gate, all {w.E} experts), numpy fp64, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this size (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(expert parallelism across GPUs is not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import moe_inputs as MI
    from mixture_experts_layer_50_amd import binding as B
    from mixture_experts_layer_50_amd.layer import LayerBuffers, backward, forward

    if not os.path.exists(B.lib_path()):
        from mixture_experts_layer_50_amd.build import build
        build()
    B.load_library()
    torch.cuda.set_device(0)
    w = MI.WORKLOADS[args.workload]
    log(f"[bench] workload {w.name}: generating inputs")
    a = MI.generate(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = {k: (torch.from_numpy(v) if k == "b" else torch.from_numpy(v).to(dt)).cuda()
           for k, v in a.items()}
    del a
    shape = B.MoEShape.make(w.T, w.d, w.E, w.k, w.I, dtype=w.dtype, gate=w.gate, e_lo=w.e_lo,
                            e_hi=w.e_end)
    buf = LayerBuffers(shape, training=w.backward)
    stream = torch.cuda.current_stream()

    def step():
        forward(shape, buf, dev["x"], dev.get("Wr"), dev.get("b"), dev["Wg"], dev["Wu"], dev["Wd"])
        if w.backward:
            backward(shape, buf, dev["dY"], dev["x"], dev.get("Wr"), dev["Wg"], dev["Wu"], dev["Wd"])

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    B.prof_enable(True)
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    B.prof_reset()
    log(f"[bench] timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    kernels = {}
    for name in B.prof_names():
        tot, n = B.prof_read(name)
        kernels[name] = {"ms_total": tot, "launches": n, "us_avg": 1000.0 * tot / max(n, 1)}
    B.prof_enable(False)

    # the same number of steps without the kernel timer (its events add gaps)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_plain = e0.elapsed_time(e1) / args.steps

    R = int(buf["offsets"][-1].item())
    El = w.E_loc
    gem = {}
    for name, (fl, by) in GEMMS.items():
        if name in kernels:
            us = kernels[name]["us_avg"]
            f, b = fl(R, w.d, w.I, El), by(R, w.d, w.I, El)
            gem[name] = {"us": round(us, 2), "tflops": round(f / us / 1e6, 1),
                         "gbs": round(b / us / 1e3, 1), "mfma_frac": round(f / us / 1e6 / PEAK_BF16_TFLOPS, 3),
                         "hbm_frac": round(b / us / 1e3 / PEAK_HBM_GBS, 3)}
    dom = max(gem, key=lambda k: kernels[k]["ms_total"])
    fl, by = GEMMS[dom]
    flops = fl(R, w.d, w.I, El)
    achieved = flops / kernels[dom]["us_avg"] / 1e6
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        ent = tr.get("kernels", {}).get(dom)
        if ent and tr.get("source_hash") == kernel_source_hash():
            traffic = ent["bytes_per_launch"]
    gemm_total_us = sum(g["us"] for g in gem.values())
    gemm_flops = sum(GEMMS[n][0](R, w.d, w.I, El) for n in gem)

    out = {
        "metric": METRIC,
        "value": round(w.T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights, N(0,1) upstream grad)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "I": w.I,
                   "gate": w.gate, "pass": "fwd+bwd" if w.backward else "fwd",
                   "routed_rows": R, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": dom},
        "grouped_gemm": {"tflops_all_six": round(gemm_flops / gemm_total_us / 1e6, 1),
                         "mfma_frac_all_six": round(gemm_flops / gemm_total_us / 1e6 / PEAK_BF16_TFLOPS, 4),
                         "kernels": gem},
        "ms_per_step_without_kernel_timer": round(ms_plain, 4),
        "wall_s_timed": round(wall, 3),
        "kernels_us_avg": {k: round(v["us_avg"], 2) for k, v in kernels.items()},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
