"""GPU parity of the small-batch forward (moe_small_fwd: the gate, then
moe_ffn_small_fwd, the batched_mm backend's counterpart: no sort, every
(token, slot) pair reads its expert's weights, the combine folded into the
down kernel): logits, routing and y against the CPU oracle, and y against the
grouped path, on the parity workloads, at decode sizes of the Qwen3 shape
(the few-token router for T <= 16), and with routing tables that hold
non-local and repeated expert ids."""
import sys

import numpy as np
import pytest
import torch

import moe_inputs as MI
import gpu_util as U
from mixture_experts_layer_50_amd import binding as B
from mixture_experts_layer_50_amd.layer import (LayerBuffers, forward_inference, forward_small,
                                                small_path_fits)
from oracle import moe_oracle as O
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

# the parity workloads within the small kernels' limit of 4096 routed pairs
SMALL_FIT = [w for w in SMALL if w.T * w.k <= B.SMALL_MAX_PAIRS]


def _announce(name):
    print(f"\n[gpu case] small-batch {name}", flush=True)
    sys.stdout.flush()


def run_small(w, dev, R_cap=0):
    s = U.shape_of(w, R_cap)
    buf = LayerBuffers(s, training=False)
    forward_small(s, buf, dev["x"], dev.get("Wr"), dev.get("b"), dev["Wg"], dev["Wu"], dev["Wd"])
    torch.cuda.synchronize()
    return s, buf


@pytest.mark.parametrize("w", SMALL_FIT, ids=[w.name for w in SMALL_FIT])
def test_small_batch_matches_oracle(w):
    _announce(w.name)
    a = MI.generate(w, parts=("x", "Wr", "b", "Wg", "Wu", "Wd"))
    f, _ = U.oracle_full(w, a)
    dev = U.upload(w, a)
    _, sb = run_small(w, dev)
    tol = U.TOL[w.dtype]
    if w.gate == "softmax_topk":
        U.check("logits", U.np64(sb["logits"]), f["logits"], 1e-5)
        U.assert_routing_well_posed(U.np64(sb["logits"]), f["logits"], w.k)
    assert np.array_equal(sb["topk_idx"].cpu().numpy(), f["idx"])
    U.check("topk_w", U.np64(sb["topk_w"]), f["g"], 1e-5)
    e = U.check("y(small)", U.np64(sb["y"]), f["y"], tol)
    # the grouped path on the same inputs agrees to the same tolerance
    _, gb = U.run_layer(w, dev, training=False)
    U.check("y(small) vs y(grouped)", U.np64(sb["y"]), U.np64(gb["y"]), tol)
    print(f"y rel err {e:.2e}")


def _oracle_y(x, idx, g, Wg, Wu, Wd, E, e_lo, e_hi):
    """The oracle's layer output for a given routing table: permute (local,
    first-occurrence slots), expert FFN, combine."""
    T, k = idx.shape
    p = O.permute(idx, x, E, e_lo, e_hi)
    f = O.expert_ffn_fwd(p["Xp"], p["offsets"], Wg, Wu, Wd)
    return O.combine(f["Yp"], p["inv"], g, T, k)


@pytest.mark.parametrize("T", [1, 2, 4, 5, 8, 16, 17, 64])
def test_decode_sizes_qwen3_shape(T):
    """Natural router at the Qwen3 shape on the first T tokens of its workload."""
    w0 = MI.WORKLOADS["qwen3_natural_fwd_T4096_d2048_E128_k8_I768"]
    w = MI.Workload(**{**w0.__dict__, "name": f"qwen3_natural_decode_T{T}", "T": T})
    _announce(w.name)
    a = MI.generate(w0, parts=("x", "Wr", "b", "Wg", "Wu", "Wd"))
    a["x"] = a["x"][:T]
    dev = U.upload(w, a)
    _, sb = run_small(w, dev)
    L, idx, g = O.route(a["x"], a["Wr"], a["b"], w.k, w.gate)
    U.check("logits", U.np64(sb["logits"]), L, 1e-5)
    U.assert_routing_well_posed(U.np64(sb["logits"]), L, w.k)
    assert np.array_equal(sb["topk_idx"].cpu().numpy(), idx)
    U.check("topk_w", U.np64(sb["topk_w"]), g, 1e-5)
    ref = _oracle_y(a["x"], idx, g, a["Wg"], a["Wu"], a["Wd"], w.E, 0, w.E)
    U.check("y(small)", U.np64(sb["y"]), ref, U.TOL["bf16"])
    _, gb = U.run_layer(w, dev, training=False)
    U.check("y(small) vs y(grouped)", U.np64(sb["y"]), U.np64(gb["y"]), U.TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_routing_table_with_foreign_and_repeated_experts(dtype):
    """A caller's routing table: slots outside the local range [4, 12) and
    repeated ids (only the first occurrence counts, as in the permute)."""
    T, d, E, k, I = 37, 128, 16, 4, 192
    w = MI.small_workload("table", T, d, E, k, I, dtype=dtype, e_lo=4, e_hi=12, seed=41,
                          backward=False)
    _announce(f"routing table {dtype}")
    a = MI.generate(w, parts=("x", "Wg", "Wu", "Wd"))
    rng = np.random.default_rng(41)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[3] = [5, 5, 5, 5]
    idx[4] = [0, 1, 2, 3]            # no local slot: y = 0
    idx[5] = [11, 4, 11, 4]
    g = rng.random((T, k)).astype(np.float32)
    dev = U.upload(w, a)
    s = U.shape_of(w)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = torch.full((T, d), float("nan"), dtype=dt, device="cuda")
    ws = torch.empty(B.workspace_size(s, "small_fwd"), dtype=torch.uint8, device="cuda")
    B.moe_ffn_small_fwd(s, dev["x"], torch.from_numpy(idx).cuda(), torch.from_numpy(g).cuda(),
                        dev["Wg"], dev["Wu"], dev["Wd"], y, ws)
    torch.cuda.synchronize()
    ref = _oracle_y(a["x"], idx, g.astype(np.float64), a["Wg"], a["Wu"], a["Wd"], E, 4, 12)
    got = U.np64(y)
    assert np.all(got[4] == 0)
    U.check("y", got, ref, U.TOL[dtype])


# the few-token router (T <= 16) at other expert counts (one to eight logits
# per lane), fp32, with a bias and on an expert slice
FEW = [
    MI.small_workload("few_T5_d256_E16_k4_I192", 5, 256, 16, 4, 192, bias_sigma=1.0, seed=71),
    MI.small_workload("few_T16_d128_E320_k6_I128", 16, 128, 320, 6, 128, bias_sigma=1.0, seed=72),
    MI.small_workload("few_T3_d512_E512_k8_I64", 3, 512, 512, 8, 64, bias_sigma=2.0, seed=73),
    MI.small_workload("few_f32_T7_d128_E64_k3_I192", 7, 128, 64, 3, 192, dtype="f32",
                      bias_sigma=1.0, seed=74, x_sigma=0.5),
    MI.small_workload("few_slice_T9_d192_E32_k4_I128_loc8_24", 9, 192, 32, 4, 128,
                      bias_sigma=3.0, e_lo=8, e_hi=24, seed=75),
    MI.small_workload("few_balanced_T6_d256_E16_k4_I192", 6, 256, 16, 4, 192, gate="balanced",
                      seed=76),
    # d = 2112 read whole by the gate/up kernel (8 active experts x 64 column
    # blocks, no K split; 66 batches of rows a lane) ...
    MI.small_workload("few_f32_T16_d2112_E8_k4_I2048", 16, 2112, 8, 4, 2048, dtype="f32",
                      bias_sigma=1.0, seed=77, x_sigma=0.5),
    # ... and A rows of width 2112 > 2048 in the down kernel (one token per pass)
    MI.small_workload("wide_I_T20_d256_E8_k2_I2112", 20, 256, 8, 2, 2112, bias_sigma=1.0,
                      seed=78),
    # fp32 with E not a multiple of 4: the final top-k kernel pads its row
    # (T*E = 1136 > 1024 keeps it out of the gate/up kernel), and the folded
    # form with an odd E
    MI.small_workload("few_f32_T16_d128_E71_k5_I64", 16, 128, 71, 5, 64, dtype="f32",
                      bias_sigma=1.0, seed=79, x_sigma=0.5),
    # too many split partials for the folded router: moe_route's few-token
    # logits and top-k, then the FFN
    MI.small_workload("few_f32_T6_d1024_E128_k4_I64", 6, 1024, 128, 4, 64, dtype="f32",
                      bias_sigma=1.0, seed=81, x_sigma=0.5),
    MI.small_workload("few_f32_T3_d192_E7_k3_I64", 3, 192, 7, 3, 64, dtype="f32",
                      bias_sigma=1.0, seed=80, x_sigma=0.5),
]


@pytest.mark.parametrize("w", FEW, ids=[w.name for w in FEW])
def test_few_token_router_and_ffn(w):
    _announce(w.name)
    a = MI.generate(w, parts=("x", "Wr", "b", "Wg", "Wu", "Wd"))
    f, _ = U.oracle_full(w, a)
    dev = U.upload(w, a)
    _, sb = run_small(w, dev)
    if w.gate == "softmax_topk":
        U.check("logits", U.np64(sb["logits"]), f["logits"], 1e-5)
        U.assert_routing_well_posed(U.np64(sb["logits"]), f["logits"], w.k)
    assert np.array_equal(sb["topk_idx"].cpu().numpy(), f["idx"])
    U.check("topk_w", U.np64(sb["topk_w"]), f["g"], 1e-5)
    U.check("y", U.np64(sb["y"]), f["y"], U.TOL[w.dtype])


def test_small_forward_repeatable_and_reuses_workspace():
    """Two calls in a row (the second with fewer tokens, the same buffers and
    workspace) give the oracle's y each time, and a repeat is bit-identical:
    the arrival counters restart at zero on every call."""
    w0 = MI.WORKLOADS["qwen3_natural_fwd_T4096_d2048_E128_k8_I768"]
    a = MI.generate(w0, parts=("x", "Wr", "b", "Wg", "Wu", "Wd"))
    w = MI.Workload(**{**w0.__dict__, "name": "qwen3_natural_decode_T16", "T": 16})
    _announce("repeat T16 then T3")
    a["x"] = a["x"][:16]
    dev = U.upload(w, a)
    s16 = U.shape_of(w)
    buf = LayerBuffers(s16, training=False)
    args = (dev["x"], dev["Wr"], dev["b"], dev["Wg"], dev["Wu"], dev["Wd"])
    forward_small(s16, buf, *args)
    y1 = buf["y"].clone()
    forward_small(s16, buf, *args)
    torch.cuda.synchronize()
    assert torch.equal(y1, buf["y"]), "repeat differs"
    L, idx, g = O.route(a["x"], a["Wr"], a["b"], w.k, w.gate)
    U.check("y(T16)", U.np64(y1), _oracle_y(a["x"], idx, g, a["Wg"], a["Wu"], a["Wd"], w.E, 0, w.E),
            U.TOL["bf16"])
    # fewer tokens through the same buffers: the first 3 rows
    s3 = U.shape_of(MI.Workload(**{**w.__dict__, "T": 3}))
    forward_small(s3, buf, dev["x"][:3], dev["Wr"], dev["b"], dev["Wg"], dev["Wu"], dev["Wd"])
    torch.cuda.synchronize()
    U.check("y(T3)", U.np64(buf["y"][:3]),
            _oracle_y(a["x"][:3], idx[:3], g[:3], a["Wg"], a["Wu"], a["Wd"], w.E, 0, w.E),
            U.TOL["bf16"])


@pytest.mark.parametrize("T", [7, 8])
def test_inference_size_rule(T):
    """forward_inference takes the small-batch call at T = 7 and the grouped
    path at T = 8 (Qwen3 shape, E_loc = 128, k = 8); both match the oracle."""
    w0 = MI.WORKLOADS["qwen3_natural_fwd_T4096_d2048_E128_k8_I768"]
    w = MI.Workload(**{**w0.__dict__, "name": f"qwen3_natural_infer_T{T}", "T": T})
    _announce(w.name)
    a = MI.generate(w0, parts=("x", "Wr", "b", "Wg", "Wu", "Wd"))
    a["x"] = a["x"][:T]
    dev = U.upload(w, a)
    s = U.shape_of(w)
    buf = LayerBuffers(s, training=False)
    assert small_path_fits(s, False) == (T <= 7)
    forward_inference(s, buf, dev["x"], dev["Wr"], dev["b"], dev["Wg"], dev["Wu"], dev["Wd"])
    torch.cuda.synchronize()
    assert ("ws_small_routed_fwd" in buf.t) == (T <= 7)
    L, idx, g = O.route(a["x"], a["Wr"], a["b"], w.k, w.gate)
    assert np.array_equal(buf["topk_idx"].cpu().numpy(), idx)
    U.check("y", U.np64(buf["y"]), _oracle_y(a["x"], idx, g, a["Wg"], a["Wu"], a["Wd"], w.E, 0, w.E),
            U.TOL["bf16"])
