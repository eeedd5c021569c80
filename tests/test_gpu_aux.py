"""Parity of the router's load-balancing auxiliary loss with the oracle on the
GPU: moe_aux_loss (loss and backward weights) and moe_route_bwd_aux (the
loss's gradient pushed through the router) called through the C ABI by the
layer, at small shapes (E from 16 to 320, fp32 and bf16) and at the full
Qwen3 natural-router shape."""
import sys

import numpy as np
import pytest
import torch

import moe_inputs as MI
import gpu_util as U
from mixture_experts_layer_50_amd.layer import LayerBuffers, backward, forward
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

CASES = [
    MI.small_workload("aux_bias_T300_d256_E16_k4_I192", 300, 256, 16, 4, 192, bias_sigma=1.0,
                      seed=61),
    MI.small_workload("aux_f32_T200_d128_E16_k3_I192", 200, 128, 16, 3, 192, dtype="f32",
                      bias_sigma=0.5, seed=62),
    MI.small_workload("aux_T500_d256_E128_k8_I256", 500, 256, 128, 8, 256, bias_sigma=1.5, seed=63),
    MI.small_workload("aux_T70_d128_E320_k6_I128", 70, 128, 320, 6, 128, bias_sigma=1.0, seed=64),
]
# the loss, its backward weights and the router gradients are fp32 outputs
# (fp32 softmax of fp32 logits, fp32 sums over the tokens), held to the fp32
# bound max|err| / max|ref| <= 1e-5 against the fp64 oracle
AUX_TOL = 1e-5


def _run(w, a, alpha, zero_dy=False):
    print(f"\n[gpu case] {w.name} alpha={alpha} zero_dy={zero_dy}", flush=True)
    sys.stdout.flush()
    dev = U.upload(w, a)
    if zero_dy:
        dev["dY"] = torch.zeros_like(dev["dY"])
    s = U.shape_of(w)
    buf = LayerBuffers(s, training=True, aux_alpha=alpha)
    forward(s, buf, dev["x"], dev.get("Wr"), dev.get("b"), dev["Wg"], dev["Wu"], dev["Wd"])
    backward(s, buf, dev["dY"], dev["x"], dev.get("Wr"), dev["Wg"], dev["Wu"], dev["Wd"])
    torch.cuda.synchronize()
    return buf


def _aux_only_router_grads(w, a, L, idx, alpha):
    """The oracle's auxiliary loss and its gradients alone (no combine term)."""
    r = O.aux_loss(L, idx, w.E, alpha)
    dL = O.aux_loss_dlogits(L, r["w"])
    zero = np.zeros(idx.shape)
    rb = O.route_bwd(a["x"], a["Wr"], idx, zero, zero, O.GATE_SOFTMAX_TOPK, dL_aux=dL)
    return r, rb


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_aux_loss_and_layer_gradients_match_oracle(w):
    alpha = 0.01
    a = MI.generate(w)
    buf = _run(w, a, alpha)
    t = buf.t
    # the kernel on the GPU's own logits and routing
    Lg, idxg = U.np64(t["logits"]), t["topk_idx"].cpu().numpy()
    rg = O.aux_loss(Lg, idxg, w.E, alpha)
    assert abs(t["aux_loss"].item() - rg["loss"]) <= AUX_TOL * abs(rg["loss"])
    U.check("aux_w", U.np64(t["aux_w"]), rg["w"], AUX_TOL)
    # end to end against the oracle's own forward and backward
    f, bw = U.oracle_full(w, a)
    assert np.array_equal(idxg, f["idx"]), "topk_idx differs"
    r, rb = _aux_only_router_grads(w, a, f["logits"], f["idx"], alpha)
    assert abs(t["aux_loss"].item() - r["loss"]) <= AUX_TOL * abs(r["loss"])
    tol = U.TOL[w.dtype]
    U.check("dlogits", U.np64(t["dlogits"]), bw["dL"] + rb["dL"], tol)
    U.check("dw_router", U.np64(t["dw_router"]), bw["dWr"] + rb["dWr"], tol)
    U.check("dbias", U.np64(t["dbias"]), bw["db"] + rb["db"], tol)
    U.check("dx", U.np64(t["dx"]), bw["dX"] + rb["dX"], tol)


@pytest.mark.parametrize("w", CASES[:3], ids=[c.name for c in CASES[:3]])
def test_aux_gradient_alone(w):
    """dY = 0 leaves only the auxiliary loss's gradient on the router (the
    expert path contributes exactly nothing), so that term is checked at full
    relative precision rather than next to the combine gradient."""
    alpha = 1.0
    a = MI.generate(w)
    buf = _run(w, a, alpha, zero_dy=True)
    t = buf.t
    L, idx = O.router_logits(a["x"], a["Wr"], a.get("b")), t["topk_idx"].cpu().numpy()
    r, rb = _aux_only_router_grads(w, a, L, idx, alpha)
    tol = U.TOL[w.dtype]
    # dlogits and dbias are fp32 outputs (fp32 softmax of fp32 logits)
    U.check("dlogits", U.np64(t["dlogits"]), rb["dL"], AUX_TOL)
    U.check("dw_router", U.np64(t["dw_router"]), rb["dWr"], tol)
    U.check("dbias", U.np64(t["dbias"]), rb["db"], AUX_TOL)
    U.check("dx", U.np64(t["dx"]), rb["dX"], tol)


def test_aux_deterministic():
    w = CASES[2]
    a = MI.generate(w)
    b1 = _run(w, a, 0.02)
    got1 = {k: b1[k].clone() for k in ("aux_loss", "aux_w", "dlogits", "dw_router", "dbias")}
    b2 = _run(w, a, 0.02)
    for k, v in got1.items():
        assert torch.equal(v, b2[k]), f"{k} differs between identical calls"


def test_full_size_qwen3_natural_aux():
    """Qwen3-30B-A3B natural router (T = 4096, E = 128, k = 8): the loss and
    the auxiliary-only router gradients (dY = 0) against the oracle."""
    w = MI.WORKLOADS["qwen3_natural_fwd_T4096_d2048_E128_k8_I768"]
    a = MI.generate(w)
    a["dY"] = np.zeros((w.T, w.d), dtype=np.float32)
    alpha = 0.5
    buf = _run(w, a, alpha)
    t = buf.t
    Lg, idxg = U.np64(t["logits"]), t["topk_idx"].cpu().numpy()
    rg = O.aux_loss(Lg, idxg, w.E, alpha)
    assert abs(t["aux_loss"].item() - rg["loss"]) <= AUX_TOL * abs(rg["loss"])
    U.check("aux_w", U.np64(t["aux_w"]), rg["w"], AUX_TOL)
    r, rb = _aux_only_router_grads(w, a, Lg, idxg, alpha)
    U.check("dlogits", U.np64(t["dlogits"]), rb["dL"], AUX_TOL)
    U.check("dw_router", U.np64(t["dw_router"]), rb["dWr"], U.TOL["bf16"])
    U.check("dbias", U.np64(t["dbias"]), rb["db"], AUX_TOL)
    U.check("dx", U.np64(t["dx"]), rb["dX"], U.TOL["bf16"])
