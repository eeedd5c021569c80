"""Benchmark of the MoE expert layer on one MI355X.

One step = one forward and one backward of the whole layer (route, permute,
grouped SwiGLU FFN, combine and the backward of each) on the Qwen3-30B-A3B
shaped workload with the balanced gate: T=4096 tokens, d=2048, E=128 experts,
k=8, I=768, bf16 storage with fp32 accumulation, seeded synthetic inputs that
are resident in HBM before the timed region.  By default the expert FFN runs
in its gathered form (the GEMMs read the permuted rows from x through the
token table; outputs bit-identical to the form with the Xp copy).

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
# of R routed rows, d, I, E_loc and T tokens.  Bytes: every operand read once,
# every output written once, bf16 (2 bytes).  The gathered forms read the
# rows of Xp from x, so their A operand is x itself (T rows, not R).
GEMMS = {
    "ffn_gateup_fwd":   (lambda R, d, I, El, T: 4 * R * d * I,
                         lambda R, d, I, El, T: 2 * (R * d + 2 * El * d * I + 2 * R * I + R * I)),
    "ffn_gateup_fwd_gather":
                        (lambda R, d, I, El, T: 4 * R * d * I,
                         lambda R, d, I, El, T: 2 * (T * d + 2 * El * d * I + 2 * R * I + R * I)),
    "ffn_down_fwd":     (lambda R, d, I, El, T: 2 * R * I * d,
                         lambda R, d, I, El, T: 2 * (R * I + El * I * d + R * d)),
    "ffn_down_dgrad":   (lambda R, d, I, El, T: 2 * R * d * I,
                         lambda R, d, I, El, T: 2 * (R * d + El * I * d + 2 * R * I + 2 * R * I)),
    "ffn_gateup_dgrad": (lambda R, d, I, El, T: 4 * R * d * I,
                         lambda R, d, I, El, T: 2 * (2 * R * I + 2 * El * d * I + R * d)),
    "ffn_down_wgrad":   (lambda R, d, I, El, T: 2 * R * I * d,
                         lambda R, d, I, El, T: 2 * (R * I + R * d + El * I * d)),
    "ffn_gateup_wgrad": (lambda R, d, I, El, T: 4 * R * d * I,
                         lambda R, d, I, El, T: 2 * (R * d + 2 * R * I + 2 * El * d * I)),
    "ffn_gateup_wgrad_gather":
                        (lambda R, d, I, El, T: 4 * R * d * I,
                         lambda R, d, I, El, T: 2 * (T * d + 2 * R * I + 2 * El * d * I)),
    # the dY form of the backward: the rows of dYp read as g * dY[t] (A or B
    # operand: dY itself, T rows)
    "ffn_down_dgrad_dy":
                        (lambda R, d, I, El, T: 2 * R * d * I,
                         lambda R, d, I, El, T: 2 * (T * d + El * I * d + 2 * R * I + 2 * R * I)),
    "ffn_down_wgrad_dy":
                        (lambda R, d, I, El, T: 2 * R * I * d,
                         lambda R, d, I, El, T: 2 * (R * I + T * d + El * I * d)),
    # the down projection with the combine in its epilogue: also reads the
    # token's rows of Yp back and writes y
    "ffn_down_fwd_combine":
                        (lambda R, d, I, El, T: 2 * R * I * d,
                         lambda R, d, I, El, T: 2 * (R * I + El * I * d + 2 * R * d + T * d)),
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_50_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(budget_s: float, dsv3_sample: bool = True):
    """The oracle (numpy fp64) timed on the host on a bounded sample of the
    workload: the same layer with the first T_s tokens (balanced gate, so every
    expert keeps an equal share of rows), each step of the layer timed on its
    own.  Also (dsv3_sample) the oracle's expert FFN, forward and backward, on
    4 of the 32 local experts of the DeepSeek-V3 rank share (1,024 rows each),
    extrapolated to all 32."""
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
        """One fwd+bwd in the oracle's own call order, each call timed."""
        x, dY = a["x"][:Ts], a["dY"][:Ts]
        t = {}

        def timed(name, fn, *args):
            t0 = time.perf_counter()
            r = fn(*args)
            t[name] = time.perf_counter() - t0
            return r

        L, idx, g = timed("route", O.route, x, a["Wr"], None, w.k, w.gate)
        p = timed("permute", O.permute, idx, x, w.E)
        f = timed("ffn_fwd", O.expert_ffn_fwd, p["Xp"], p["offsets"], a["Wg"], a["Wu"], a["Wd"])
        timed("combine", O.combine, f["Yp"], p["inv"], g, Ts, w.k)
        dYp, dG = timed("combine_bwd", O.combine_bwd, dY, f["Yp"], p["inv"], g, Ts, w.k)
        fb = timed("ffn_bwd", O.expert_ffn_bwd, p["Xp"], p["offsets"], a["Wg"], a["Wu"], a["Wd"],
                   f["Hg"], f["Hu"], f["A"], dYp)
        timed("permute_bwd", O.permute_bwd, fb["dXp"], p["inv"], Ts, w.k)
        timed("route_bwd", O.route_bwd, x, a["Wr"], idx, g, dG, w.gate)
        return sum(t.values()), t

    t_probe, _ = step(512)
    est_full = t_probe * w.T / 512  # overestimates: the probe carries fixed costs
    Ts = w.T if est_full <= 2 * budget_s else int(max(512, 512 * budget_s / t_probe)) // 256 * 256
    dt, steps = step(Ts)
    out = {"value": round(Ts / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"one fwd+bwd of the layer on the first {Ts} of {w.T} tokens "
                     f"(balanced gate, all {w.E} experts), numpy fp64, {dt:.1f} s",
           "step_s": {k: round(v, 4) for k, v in steps.items()}}
    del a
    if dsv3_sample:
        wd = MI.WORKLOADS["dsv3_ep8_rank_fwdbwd_T32768_d7168_E256_loc32_k8_I2048"]
        experts = [0, 1, 17, 31]
        ad = MI.generate(wd, parts=("x", "dY"))
        P = wd.E // wd.k
        t_ffn = 0.0
        for e in experts:
            tok = np.arange(e, wd.T, P)  # the balanced gate sends tokens t = e mod P to expert e
            Xe = ad["x"][tok]
            Wg, Wu, Wd = (MI.expert_weights(wd, n, [e]) for n in ("Wg", "Wu", "Wd"))
            one = np.array([0, len(tok)])
            t0 = time.perf_counter()
            fe = O.expert_ffn_fwd(Xe, one, Wg, Wu, Wd)
            O.expert_ffn_bwd(Xe, one, Wg, Wu, Wd, fe["Hg"], fe["Hu"], fe["A"],
                             ad["dY"][tok] / wd.k)
            t_ffn += time.perf_counter() - t0
        scale = wd.E_loc / len(experts)
        out["dsv3_rank_share_ffn"] = {
            "kind": "oracle, extrapolated", "experts_timed": experts,
            "rows_per_expert": wd.T * wd.k // wd.E, "seconds_timed": round(t_ffn, 2),
            "extrapolation_factor": scale,
            "ffn_fwdbwd_s_extrapolated": round(t_ffn * scale, 2),
            "note": "expert FFN forward and backward only (the GEMMs: over 99% of the layer's "
                    "flops) of 4 sampled local experts, times 8 for the 32 local experts"}
    return out


# GEMM roles: the last template argument of the GEMM kernels
ROLE_NAMES = {0: "route_logits", 1: "ffn_gateup_fwd", 2: "ffn_down_fwd", 3: "ffn_down_dgrad",
              4: "ffn_gateup_dgrad", 5: "ffn_down_wgrad", 6: "ffn_gateup_wgrad", 7: "route_bwd_dw",
              8: "route_bwd_dx", 9: "ffn_gateup_fwd_gather", 10: "ffn_gateup_wgrad_gather",
              11: "ffn_down_fwd_combine", 12: "ffn_down_dgrad_dy"}


def gemm_role_of(kernel_name: str, dy_form: bool = False):
    """The GEMM role of a kernel from its name; dy_form: the run used
    moe_combine_ffn_bwd_gather, whose down weight gradient launches the strip
    kernel's dY form and then the role's tile kernel."""
    if "gemm_bf16" not in kernel_name:
        return None
    args = kernel_name.split("<", 1)[1].split(">", 1)[0].split(",")
    if args[0].strip() == "true":  # the strip kernel's dY form
        return "ffn_down_wgrad_dy"
    role = ROLE_NAMES.get(int(args[-1]))
    return "ffn_down_wgrad_dy" if dy_form and role == "ffn_down_wgrad" else role


def summarize_pmc(fetch_csv: str, write_csv: str, calib_mib: int) -> dict:
    """HBM bytes per launch of each layer kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for a fill (writes) and a sum (reads) of calib_mib MiB."""
    import csv
    import collections

    def per_kernel(path, counter):
        vals = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    calib = calib_mib * (1 << 20)
    rd = [v for k, v in fetch.items() if "reduce" in k.lower()]
    wr = [v for k, v in write.items() if "FillFunctor" in k]
    f_read = calib / (max(rd[0]) * 1024) if rd else 1.0
    f_write = calib / (max(wr[0]) * 1024) if wr else 1.0
    out = {"source_hash": kernel_source_hash(), "calibration": {
        "read_factor": round(f_read, 4), "write_factor": round(f_write, 4),
        "calib_bytes": calib}, "kernels": {}, "raw_kib_per_dispatch": {}}
    dy_form = any(gemm_role_of(k) == "ffn_down_wgrad_dy" for k in fetch)
    for k in fetch:
        f = sum(fetch[k]) / len(fetch[k])
        w_ = sum(write.get(k, [0.0])) / max(len(write.get(k, [])), 1)
        out["raw_kib_per_dispatch"][k] = {"FETCH_SIZE": round(f, 1), "WRITE_SIZE": round(w_, 1)}
        role = gemm_role_of(k, dy_form)
        if role:
            # a role may launch two kernels (the weight gradients' strip
            # kernel and tile kernel): its bytes per call are their sum
            ent = out["kernels"].setdefault(role, {"bytes_per_launch": 0, "read_bytes": 0,
                                                   "write_bytes": 0})
            ent["read_bytes"] += int(f * 1024 * f_read)
            ent["write_bytes"] += int(w_ * 1024 * f_write)
            ent["bytes_per_launch"] = ent["read_bytes"] + ent["write_bytes"]
    return out


def timed_steps(step, steps: int, warmup: int):
    """Median / min / p90 / mean of per-step times (HIP events around each step)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return {"median": round(t[len(t) // 2], 4), "min": round(t[0], 4),
            "p90": round(t[min(len(t) - 1, int(0.9 * len(t)))], 4),
            "mean": round(sum(t) / len(t), 4)}


def graph_step_ms(step, replays: int):
    """GPU time per call of step, captured once in a HIP graph and replayed
    `replays` times between two events (no host enqueue in the span)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / replays
    del g
    return ms


def form_buffers(shape, training: bool, form: str, **kw):
    """The layer's buffers for one FFN form: plain (the permute writes Xp),
    gather (the FFN reads x through the token table), fused (gather, with the
    combine in the down projection's epilogue), dy (gather, with the
    backward's dYp rows formed from dY inside the kernels)."""
    from mixture_experts_layer_50_amd.layer import LayerBuffers
    return LayerBuffers(shape, training=training, gather=form != "plain", fused=form == "fused",
                        dy_form=form == "dy", **kw)


def kernel_averages(step, B, n: int):
    """Per-kernel averages (us) over n instrumented steps."""
    import torch
    B.prof_select(None)
    B.prof_enable(True)
    B.prof_reset()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    res = {}
    for name in B.prof_names():
        tot, cnt = B.prof_read(name)
        res[name] = round(1000.0 * tot / max(cnt, 1), 2)
    B.prof_enable(False)
    return res


def secondary_workloads(B, dev, w_main, gather, which="all"):
    """The main workload with the other FFN form (Xp materialised by the
    permute, or read from x through the token table); fwd+bwd of the natural
    softmax top-k router at the Qwen3 shape (same tokens and expert weights as
    the main workload, router weights and bias from the natural workload's
    recipe), also with the router's balancing loss; decode-sized forwards of
    the small-batch and grouped paths; and fwd+bwd of one rank's share of the
    DeepSeek-V3 shape (expert weights drawn on the GPU with the same
    distribution as the recipe).  `which`: a comma-separated subset of
    other_ffn, natural, natural_aux, small, dsv3 (or 'all')."""
    import numpy as np
    import torch
    import moe_inputs as MI
    from mixture_experts_layer_50_amd.layer import LayerBuffers, backward, forward, forward_small

    out = {}
    want = set(which.split(",")) if which != "all" else {"other_ffn", "fwd", "natural",
                                                          "natural_aux", "small", "dsv3"}
    if "fwd" in want:
        # forward only, inference (no H saved for a backward pass): the balanced
        # gate on the main workload's tensors (the work does not depend on the
        # values: every expert gets T*k/E rows), and the natural router on the
        # natural workload's own tokens, router weights and bias (its routing:
        # 40 empty experts, largest group 3,275 rows)
        shape_b = B.MoEShape.make(w_main.T, w_main.d, w_main.E, w_main.k, w_main.I,
                                  dtype=w_main.dtype, gate="balanced")
        buf = form_buffers(shape_b, False, gather)

        def step_fwd_b():
            forward(shape_b, buf, dev["x"], None, None, dev["Wg"], dev["Wu"], dev["Wd"])

        st = timed_steps(step_fwd_b, 20, 3)
        out["balanced_fwd_inference"] = {
            "workload": "qwen3_balanced_fwd_T4096_d2048_E128_k8_I768 (shapes and routing; "
                        "tensors of the main workload)",
            "tokens_per_s": round(w_main.T / (st["median"] / 1e3), 1), "step_ms": st,
            "kernels_us_avg": kernel_averages(step_fwd_b, B, 5)}
        del buf
        w3 = MI.WORKLOADS["qwen3_natural_fwd_T4096_d2048_E128_k8_I768"]
        a3 = MI.generate(w3, parts=("x", "Wr", "b"))
        x3 = torch.from_numpy(a3["x"]).to(torch.bfloat16).cuda()
        Wr3 = torch.from_numpy(a3["Wr"]).to(torch.bfloat16).cuda()
        b3 = torch.from_numpy(a3["b"]).cuda()
        shape_n = B.MoEShape.make(w3.T, w3.d, w3.E, w3.k, w3.I, dtype="bf16", gate="softmax_topk")
        buf = form_buffers(shape_n, False, gather)

        def step_fwd_n():
            forward(shape_n, buf, x3, Wr3, b3, dev["Wg"], dev["Wu"], dev["Wd"])

        st = timed_steps(step_fwd_n, 20, 3)
        counts = np.diff(buf["offsets"].cpu().numpy())
        out["natural_fwd_inference"] = {
            "workload": "qwen3_natural_fwd_T4096_d2048_E128_k8_I768 (its tokens, router weights "
                        "and bias; expert weights of the main workload)",
            "tokens_per_s": round(w3.T / (st["median"] / 1e3), 1), "step_ms": st,
            "max_group_rows": int(counts.max()), "empty_experts": int((counts == 0).sum()),
            "kernels_us_avg": kernel_averages(step_fwd_n, B, 5)}
        del buf, x3, Wr3, b3
    if "other_ffn" in want:  # the main workload, the FFN forms the main run did not use
        shape = B.MoEShape.make(w_main.T, w_main.d, w_main.E, w_main.k, w_main.I,
                                dtype=w_main.dtype, gate=w_main.gate)
        for form in ("plain", "gather", "fused", "dy"):
            if form == gather:
                continue
            buf = form_buffers(shape, True, form)

            def step_other():
                forward(shape, buf, dev["x"], None, None, dev["Wg"], dev["Wu"], dev["Wd"])
                backward(shape, buf, dev["dY"], dev["x"], None, dev["Wg"], dev["Wu"], dev["Wd"])

            st = timed_steps(step_other, 10, 3)
            key = {"plain": "plain", "gather": "gathered", "fused": "fused", "dy": "dy_form"}[form]
            out[key + "_ffn_fwdbwd"] = {
                "workload": w_main.name, "ffn": form,
                "tokens_per_s": round(w_main.T / (st["median"] / 1e3), 1), "step_ms": st,
                "kernels_us_avg": kernel_averages(step_other, B, 3)}
            del buf
    wn = MI.WORKLOADS["qwen3_natural_fwd_T4096_d2048_E128_k8_I768"]
    r = MI.generate(wn, parts=["Wr", "b"])
    Wr = torch.from_numpy(r["Wr"]).to(torch.bfloat16).cuda()
    bias = torch.from_numpy(r["b"]).cuda()
    shape = B.MoEShape.make(wn.T, wn.d, wn.E, wn.k, wn.I, dtype="bf16", gate="softmax_topk")
    if "natural" in want:  # natural router, Qwen3 shape
        buf = form_buffers(shape, True, gather)

        def step_nat():
            forward(shape, buf, dev["x"], Wr, bias, dev["Wg"], dev["Wu"], dev["Wd"])
            backward(shape, buf, dev["dY"], dev["x"], Wr, dev["Wg"], dev["Wu"], dev["Wd"])

        st = timed_steps(step_nat, 10, 3)
        counts = np.diff(buf["offsets"].cpu().numpy())
        out["natural_router_fwdbwd"] = {
            "workload": "qwen3_natural_fwdbwd_T4096_d2048_E128_k8_I768 (router bias N(0,1.5))",
            "tokens_per_s": round(wn.T / (st["median"] / 1e3), 1), "step_ms": st,
            "max_group_rows": int(counts.max()), "empty_experts": int((counts == 0).sum()),
            "kernels_us_avg": kernel_averages(step_nat, B, 3)}
        del buf
    if "natural_aux" in want:  # the same with the balancing loss (alpha 0.01)
        buf = form_buffers(shape, True, gather, aux_alpha=0.01)

        def step_nat_aux():
            forward(shape, buf, dev["x"], Wr, bias, dev["Wg"], dev["Wu"], dev["Wd"])
            backward(shape, buf, dev["dY"], dev["x"], Wr, dev["Wg"], dev["Wu"], dev["Wd"])

        st = timed_steps(step_nat_aux, 10, 3)
        ka = kernel_averages(step_nat_aux, B, 3)
        out["natural_router_aux_fwdbwd"] = {
            "workload": "qwen3_natural_fwdbwd_T4096_d2048_E128_k8_I768 + balancing loss (alpha 0.01)",
            "tokens_per_s": round(wn.T / (st["median"] / 1e3), 1), "step_ms": st,
            "aux_loss": float(buf["aux_loss"].item()),
            "kernels_us_avg": {k: v for k, v in ka.items() if k.startswith(("aux", "route"))}}
        del buf
    if "small" in want:  # decode-sized batches, natural router, forward only
        out["small_batch_fwd"] = {
            "note": "us per forward; *_us: HIP events around eager calls (host enqueue "
                    "included when it is the longer), *_graph_us: the same calls replayed "
                    "from a HIP graph (GPU time); the size rule takes the small call for "
                    "2*T*k < E_loc (T <= 7 here)"}
        for Ts in (1, 2, 4, 8, 16, 64):
            shape_s = B.MoEShape.make(Ts, wn.d, wn.E, wn.k, wn.I, dtype="bf16",
                                      gate="softmax_topk")
            xs = dev["x"][:Ts].contiguous()
            bs = LayerBuffers(shape_s, training=False)
            bg = LayerBuffers(shape_s, training=False, gather=True)

            def step_small():
                forward_small(shape_s, bs, xs, Wr, bias, dev["Wg"], dev["Wu"], dev["Wd"])

            def step_grouped():
                forward(shape_s, bg, xs, Wr, bias, dev["Wg"], dev["Wu"], dev["Wd"])

            ss = timed_steps(step_small, 50, 5)
            sg = timed_steps(step_grouped, 50, 5)
            out["small_batch_fwd"][f"T{Ts}"] = {
                "small_us": round(1000 * ss["median"], 1),
                "grouped_us": round(1000 * sg["median"], 1),
                "small_graph_us": round(1000 * graph_step_ms(step_small, 50), 1),
                "grouped_graph_us": round(1000 * graph_step_ms(step_grouped, 50), 1),
                "small_kernels_us_avg": kernel_averages(step_small, B, 5)}
            del bs, bg
    if "dsv3" in want:  # one rank of eight at the DeepSeek-V3 shape, balanced gate
        wd = MI.WORKLOADS["dsv3_ep8_rank_fwdbwd_T32768_d7168_E256_loc32_k8_I2048"]
        g = torch.Generator(device="cuda").manual_seed(wd.seed)
        El = wd.E_loc

        def rnd(*sh, sigma):
            return (torch.randn(*sh, device="cuda", generator=g) * sigma).to(torch.bfloat16)

        d5 = {"x": rnd(wd.T, wd.d, sigma=wd.x_sigma), "Wg": rnd(El, wd.d, wd.I, sigma=wd.w_sigma),
              "Wu": rnd(El, wd.d, wd.I, sigma=wd.w_sigma),
              "Wd": rnd(El, wd.I, wd.d, sigma=wd.w_sigma),
              "dY": rnd(wd.T, wd.d, sigma=wd.dy_sigma)}
        shape_d = B.MoEShape.make(wd.T, wd.d, wd.E, wd.k, wd.I, dtype="bf16", gate="balanced",
                                  e_lo=wd.e_lo, e_hi=wd.e_end)
        buf = form_buffers(shape_d, True, gather)

        def step_ds():
            forward(shape_d, buf, d5["x"], None, None, d5["Wg"], d5["Wu"], d5["Wd"])
            backward(shape_d, buf, d5["dY"], d5["x"], None, d5["Wg"], d5["Wu"], d5["Wd"])

        st = timed_steps(step_ds, 5, 2)
        ker = kernel_averages(step_ds, B, 2)
        R = int(buf["offsets"][-1].item())
        gem_us = sum(ker[n] for n in GEMMS if n in ker)
        gem_fl = sum(GEMMS[n][0](R, wd.d, wd.I, El, wd.T) for n in GEMMS if n in ker)
        out["dsv3_rank_share_fwdbwd"] = {
            "workload": wd.name, "routed_rows": R,
            "tokens_per_s": round(wd.T / (st["median"] / 1e3), 1), "step_ms": st,
            "grouped_gemm_tflops": round(gem_fl / gem_us / 1e6, 1),
            "grouped_gemm_mfma_frac": round(gem_fl / gem_us / 1e6 / PEAK_BF16_TFLOPS, 4),
            "kernels_us_avg": ker}
        del buf, d5
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--pass", dest="pass_", choices=("default", "fwd", "fwdbwd"), default="default",
                    help="run the workload forward only or forward+backward (default: as the "
                         "workload is defined)")
    ap.add_argument("--ffn", choices=("dy", "gather", "plain", "fused"), default="dy",
                    help="gather: the FFN reads the rows of Xp from x through the token table "
                         "(no Xp buffer); plain: the permute writes Xp; fused: gather, and the "
                         "combine runs in the down projection's epilogue; dy: gather, with the "
                         "combine backward inside the FFN backward (dYp written only where a "
                         "kernel reads it, else its rows formed from dY inside the kernels)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the natural-router and DeepSeek-V3 rank-share timings")
    ap.add_argument("--secondary", default="all",
                    help="comma-separated secondary timings to run (other_ffn, natural, "
                         "natural_aux, small, dsv3) or 'all'")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--calib-mib", type=int, default=0,
                    help="also run a fill and a sum of this size (HBM counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        res = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.calib_mib or 1024)
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(res, fh, indent=1)
        print(json.dumps(res["kernels"]))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
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
    if args.pass_ != "default" and (args.pass_ == "fwdbwd") != w.backward:
        w = MI.Workload(**{**w.__dict__, "backward": args.pass_ == "fwdbwd"})
    log(f"[bench] workload {w.name} ({'fwd+bwd' if w.backward else 'fwd'}): generating inputs")
    a = MI.generate(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = {k: (torch.from_numpy(v) if k == "b" else torch.from_numpy(v).to(dt)).cuda()
           for k, v in a.items()}
    del a
    shape = B.MoEShape.make(w.T, w.d, w.E, w.k, w.I, dtype=w.dtype, gate=w.gate, e_lo=w.e_lo,
                            e_hi=w.e_end)
    gather = args.ffn  # the FFN form: dy, gather, plain or fused
    torch.cuda.synchronize()
    inputs_bytes = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    buf = form_buffers(shape, w.backward, gather)
    stream = torch.cuda.current_stream()

    def step():
        forward(shape, buf, dev["x"], dev.get("Wr"), dev.get("b"), dev["Wg"], dev["Wu"], dev["Wd"])
        if w.backward:
            backward(shape, buf, dev["dY"], dev["x"], dev.get("Wr"), dev["Wg"], dev["Wu"], dev["Wd"])

    if args.calib_mib:
        # HBM counter calibration: a fill that writes, and a sum that reads,
        # exactly calib_mib MiB (their FETCH_SIZE / WRITE_SIZE give the scale)
        n = args.calib_mib * (1 << 20) // 4
        t = torch.ones(n, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        t.sum()
        torch.cuda.synchronize()
        del t

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # calibration (untimed): three steps with every kernel on the HIP-event
    # timer to find the dominant grouped GEMM (the slowest on their sum: two
    # GEMMs within a few per cent of each other would swap on one step)
    B.prof_select(None)
    B.prof_enable(True)
    B.prof_reset()
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    calib = {n: B.prof_read(n)[0] for n in B.prof_names()}
    dom = max((n for n in calib if n in GEMMS), key=lambda n: calib[n])
    # timed region: only the dominant kernel carries HIP events (recorded on
    # the stream it is launched on), so other kernels run back to back
    B.prof_select([dom])
    B.prof_reset()
    log(f"[bench] timing {args.steps} steps (event-timed kernel: {dom})")
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
    dom_ms, dom_n = B.prof_read(dom)
    # every kernel's average, from an instrumented pass after the timed region
    B.prof_select(None)
    B.prof_reset()
    for _ in range(max(3, args.steps // 4)):
        step()
    torch.cuda.synchronize()
    kernels = {}
    for name in B.prof_names():
        tot, n = B.prof_read(name)
        kernels[name] = {"us_avg": 1000.0 * tot / max(n, 1), "launches": n}
    kernels[dom] = {"us_avg": 1000.0 * dom_ms / max(dom_n, 1), "launches": dom_n}
    B.prof_enable(False)

    peak_bytes = torch.cuda.max_memory_allocated()
    # the token kernels (route, sort, combine and their backwards) with the
    # memory-side cache flushed before every step: a 512 MiB buffer is
    # rewritten between steps, so the step's first kernels find none of the
    # previous step's data in the 256 MB MALL
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    B.prof_enable(True)
    B.prof_select(None)
    B.prof_reset()
    for i in range(5):
        flush.fill_(i)
        step()
    torch.cuda.synchronize()
    flushed = {}
    for name in B.prof_names():
        if name in GEMMS:
            continue
        tot, n = B.prof_read(name)
        flushed[name] = round(1000.0 * tot / max(n, 1), 2)
    B.prof_enable(False)
    del flush

    R = int(buf["offsets"][-1].item())
    El = w.E_loc
    gem = {}
    for name, (fl, by) in GEMMS.items():
        if name in kernels:
            us = kernels[name]["us_avg"]
            f, b = fl(R, w.d, w.I, El, w.T), by(R, w.d, w.I, El, w.T)
            gem[name] = {"us": round(us, 2), "tflops": round(f / us / 1e6, 1),
                         "gbs": round(b / us / 1e3, 1), "mfma_frac": round(f / us / 1e6 / PEAK_BF16_TFLOPS, 3),
                         "hbm_frac": round(b / us / 1e3 / PEAK_HBM_GBS, 3)}
    fl, by = GEMMS[dom]
    flops, nbytes = fl(R, w.d, w.I, El, w.T), by(R, w.d, w.I, El, w.T)
    # the dominant kernel's bound by the roofline model: HBM when its
    # algorithmic bytes take longer at peak bandwidth than its flops at peak
    # MFMA rate (intensity below the ridge point), else MFMA
    hbm_bound = nbytes / PEAK_HBM_GBS > flops / PEAK_BF16_TFLOPS / 1e3
    dom_us = kernels[dom]["us_avg"]
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(nbytes / dom_us / 1e3, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / dom_us / 1e6, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        ent = tr.get("kernels", {}).get(dom)
        if ent and tr.get("source_hash") == kernel_source_hash():
            traffic = ent["bytes_per_launch"]
    gemm_total_us = sum(g["us"] for g in gem.values())
    gemm_flops = sum(GEMMS[n][0](R, w.d, w.I, El, w.T) for n in gem)

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
                   "routed_rows": R, "ffn": args.ffn, "parallelism": "single GPU"},
        "roofline": {**roof, "traffic": traffic, "kernel": dom,
                     "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                     "mfma_tflops": round(flops / dom_us / 1e6, 1)},
        "grouped_gemm": {"tflops_all_six": round(gemm_flops / gemm_total_us / 1e6, 1),
                         "mfma_frac_all_six": round(gemm_flops / gemm_total_us / 1e6 / PEAK_BF16_TFLOPS, 4),
                         "kernels": gem},
        "wall_s_timed": round(wall, 3),
        "peak_device_memory": {"bytes": int(peak_bytes), "inputs_bytes": int(inputs_bytes),
                               "layer_buffers_bytes": int(peak_bytes - inputs_bytes),
                               "what": "torch.cuda.max_memory_allocated over the warm-up and "
                                       "timed steps (inputs: x, weights, upstream gradient)"},
        "token_kernels_us_mall_flushed": flushed,
        "kernels_us_avg": {k: round(v["us_avg"], 2) for k, v in kernels.items()},
    }
    out["step_ms_stats"] = timed_steps(step, max(5, args.steps), 2)
    if not args.no_secondary and w.name == WORKLOAD:
        log("[bench] natural-router and DeepSeek-V3 rank-share timings")
        out["secondary"] = secondary_workloads(B, dev, w, gather, args.secondary)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
