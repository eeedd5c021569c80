"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer outputs (routing indices, group offsets, permutation, inverse map)
must be bit-exact; the permuted activations are exact copies; floating-point
outputs must satisfy max|err| / max|ref| <= 2e-2 (bf16 storage, fp32
accumulation) or 1e-5 (fp32), per tensor and per expert slice of each weight
gradient."""
import sys

import numpy as np
import pytest
import torch

import moe_inputs as MI
from oracle import moe_oracle as O
import gpu_util as U

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"\n[gpu case] {name}", flush=True)
    sys.stdout.flush()


SMALL = [
    # name, shape and routing; several tiles and ragged tails
    MI.small_workload("natural_bias_T300_d256_E16_k4_I192", 300, 256, 16, 4, 192, bias_sigma=1.0, seed=21),
    MI.small_workload("balanced_T1024_d512_E8_k2_I256", 1024, 512, 8, 2, 256, gate="balanced", seed=22),
    MI.small_workload("ep_slice_T517_d256_E32_k4_I128_loc8_24", 517, 256, 32, 4, 128, bias_sigma=3.0,
                      e_lo=8, e_hi=24, seed=23),
    MI.small_workload("k1_T129_d64_E8_k1_I64", 129, 64, 8, 1, 64, bias_sigma=0.5, seed=24),
    MI.small_workload("kE_T70_d128_E8_k8_I64", 70, 128, 8, 8, 64, seed=25),
    MI.small_workload("skewed_T640_d192_E64_k6_I320", 640, 192, 64, 6, 320, bias_sigma=2.5, seed=26),
    MI.small_workload("f32_natural_T200_d128_E16_k3_I192", 200, 128, 16, 3, 192, dtype="f32",
                      bias_sigma=1.0, seed=27, x_sigma=0.5),
    # expert width >= 768: the wide tile of the dSwiGLU GEMM, ragged groups
    MI.small_workload("wide_I_T300_d128_E8_k2_I1536", 300, 128, 8, 2, 1536, bias_sigma=1.0, seed=28),
    MI.small_workload("wide_I_T260_d192_E8_k2_I768", 260, 192, 8, 2, 768, bias_sigma=1.0, seed=41),
    # 104 row tiles x 3 wide column tiles: more tiles than compute units, a
    # partial second wave
    MI.small_workload("tail_split_T3200_d64_E8_k8_I768", 3200, 64, 8, 8, 768, bias_sigma=1.0,
                      seed=43),
    # 512 experts: the sort's per-block histograms at their largest (every
    # scatter workgroup scans 512 experts' counts over all blocks)
    MI.small_workload("many_experts_T1500_d64_E512_k4_I64", 1500, 64, 512, 4, 64, bias_sigma=2.0,
                      seed=44),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_layer_fwd_bwd(w):
    _announce(w.name)
    a = MI.generate(w)
    f, bw = U.oracle_full(w, a)
    if w.gate == "softmax_topk":
        s = -np.sort(-f["logits"], axis=1)
        if w.k < w.E:
            assert (s[:, w.k - 1] - s[:, w.k]).min() > 1e-4, "seed gives a near-tie"
    s, buf = U.run_layer(w, U.upload(w, a))
    errs = U.compare_full(w, a, buf, f, bw)
    print({k: f"{v:.2e}" for k, v in errs.items()})


def test_tiny_fp32_workload_forward():
    w = MI.WORKLOADS["tiny_f32_T64_d128_E8_k2_I256"]
    _announce(w.name)
    a = MI.generate(w)
    f, _ = U.oracle_full(w, {k: v for k, v in a.items() if k != "dY"})
    s, buf = U.run_layer(w, U.upload(w, a), training=False)
    errs = U.compare_full(w, a, buf, f, None)
    print({k: f"{v:.2e}" for k, v in errs.items()})


def test_capacity_drop():
    w = MI.small_workload("cap_T256_d128_E8_k2_I128", 256, 128, 8, 2, 128, bias_sigma=1.0, seed=31)
    _announce(w.name)
    a = MI.generate(w)
    cap = 301
    f, bw = U.oracle_full(w, a, R_cap=cap)
    assert f["offsets"][-1] == cap and (f["inv"] < 0).sum() == 512 - cap
    s, buf = U.run_layer(w, U.upload(w, a), R_cap=cap)
    U.compare_full(w, a, buf, f, bw)


def test_deterministic_and_no_unwritten_outputs():
    w = SMALL[2]
    _announce("determinism+poison " + w.name)
    a = MI.generate(w)
    dev = U.upload(w, a)
    s, b1 = U.run_layer(w, dev, poison=True)
    _, b2 = U.run_layer(w, dev, poison=True)
    R = int(b1["offsets"][-1].item())
    rows_cap = s.rows_cap
    for name, t1 in b1.t.items():
        if t1 is None or name.startswith("ws_"):
            continue
        t2 = b2.t[name]
        if name in ("perm", "xp", "h", "a", "yp", "dyp", "dxp"):
            t1, t2 = t1[:R], t2[:R]
        assert torch.equal(t1.view(torch.uint8) if t1.dtype != torch.int32 else t1,
                           t2.view(torch.uint8) if t2.dtype != torch.int32 else t2), name
        if t1.is_floating_point():
            assert torch.isfinite(t1.float()).all(), f"{name} has unwritten (NaN) entries"
    assert R < rows_cap
    assert torch.isnan(b1["yp"][R:].float()).all(), "rows past the routed count were written"


@pytest.mark.parametrize("name", ["qwen3_balanced_fwd_T4096_d2048_E128_k8_I768"])
def test_full_size_balanced_forward(name):
    w = MI.WORKLOADS[name]
    _announce(name)
    a = MI.generate(w, parts=("x", "Wr", "Wg", "Wu", "Wd"))
    s, buf = U.run_layer(w, U.upload(w, a), training=False)
    # balanced gate: closed-form permutation
    P = w.E // w.k
    offs = buf["offsets"].cpu().numpy()
    assert (np.diff(offs) == w.T * w.k // w.E).all()
    perm = buf["perm"].cpu().numpy()
    m = np.arange(w.T // P)
    for e in (0, 5, 16, 127):
        assert (perm[offs[e]:offs[e + 1]] == ((e % P) + m * P) * w.k + e // P).all()
    tokens = np.r_[0:8, 1000:1004, 4090:4096]
    U.compare_sampled(w, a, buf, tokens, experts=[])


def test_full_size_natural_forward():
    w = MI.WORKLOADS["qwen3_natural_fwd_T4096_d2048_E128_k8_I768"]
    _announce(w.name)
    a = MI.generate(w, parts=("x", "Wr", "b", "Wg", "Wu", "Wd"))
    L = O.router_logits(a["x"], a["Wr"], a["b"])
    s_, buf = U.run_layer(w, U.upload(w, a), training=False)
    # no selection can flip: every token's top-k gap exceeds twice the largest
    # GPU-vs-oracle logit error (so bit-exact routing is well posed)
    gap, err = U.assert_routing_well_posed(U.np64(buf["logits"]), L, w.k)
    print(f"smallest top-k gap {gap:.2e}, largest logit error {err:.2e}")
    counts = np.diff(buf["offsets"].cpu().numpy())
    print("empty experts", int((counts == 0).sum()), "max group", int(counts.max()))
    assert (counts == 0).any() and counts.max() > 1000
    U.compare_sampled(w, a, buf, np.r_[0:16, 2048:2056, 4088:4096], experts=[])


def test_full_size_balanced_fwd_bwd():
    w = MI.WORKLOADS["qwen3_balanced_fwdbwd_T4096_d2048_E128_k8_I768"]
    _announce(w.name)
    a = MI.generate(w)
    s, buf = U.run_layer(w, U.upload(w, a))
    U.compare_sampled(w, a, buf, np.r_[0:8, 777, 3000:3004, 4095], experts=[0, 1, 63, 127])


def test_full_size_natural_fwd_bwd():
    """Natural router at the Qwen3 shape, forward and backward, every output
    element by element against the oracle's full fwd+bwd (including the
    router's weight and bias gradients over all 4,096 tokens)."""
    w = MI.WORKLOADS["qwen3_natural_fwd_T4096_d2048_E128_k8_I768"]
    w = MI.Workload(**{**w.__dict__, "name": w.name + "_bwd", "backward": True})
    _announce(w.name)
    a = MI.generate(w)
    s, buf = U.run_layer(w, U.upload(w, a))
    counts = np.diff(buf["offsets"].cpu().numpy())
    assert counts.min() == 0 and counts.max() > 1000
    f, bw = U.oracle_full(w, a)
    errs = U.compare_full(w, a, buf, f, bw)
    print({k: f"{v:.2e}" for k, v in errs.items()})


def test_full_size_dsv3_rank_share():
    w = MI.WORKLOADS["dsv3_ep8_rank_fwdbwd_T32768_d7168_E256_loc32_k8_I2048"]
    _announce(w.name)
    a = MI.generate(w)
    s, buf = U.run_layer(w, U.upload(w, a))
    offs = buf["offsets"].cpu().numpy()
    assert (np.diff(offs) == 1024).all() and offs[-1] == 32768
    U.compare_sampled(w, a, buf, np.r_[0:4, 32764:32768], experts=[0, 31])
    # expert 0's GEMMs element by element against their rounding bound on the
    # bf16 operands they read (K = 7168, 2048 and 1024: the long K loops)
    xp, h, act, yp, dyp = (U.np64(buf[n][:1024]) for n in ("xp", "h", "a", "yp", "dyp"))
    U.check_rounding_bound("h[0]", h, xp, np.concatenate([a["Wg"][0], a["Wu"][0]], 1))
    U.check_rounding_bound("yp[0]", yp, act, a["Wd"][0])
    U.check_rounding_bound("dw_down[0]", U.np64(buf["dw_down"][0]), act.T, dyp)
