"""GPU parity of the expert weight gradients on both of their paths: the
strip kernel, taken when every local expert has at most 256 rows, and the
tile kernel, taken when one expert has more (the choice is made on the
device from the group offsets).  Group sizes are set exactly by a routing
table handed in by the caller: 256-row groups (one whole K block), empty
groups, ragged ones, and a single 257-row group that moves every expert to
the tile kernel.  The output rows (d = 320) end in a partial 256-row block,
the gate/up gradient has an odd number of 128-column tiles (2I = 384) and
the down gradient a partial last tile (d = 320).  Checked against the
oracle's backward, expert by expert; and the MFMA GEMMs (the gate/up
forward and the down weight gradient on both paths) element by element
against the rounding bound of a bf16 result of an fp32 sum, recomputed from
the bf16 operands the kernels read."""
import sys

import numpy as np
import pytest
import torch

import moe_inputs as MI
import gpu_util as U
from mixture_experts_layer_50_amd import binding as B
from mixture_experts_layer_50_amd.layer import LayerBuffers
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

SIZES = {
    "strip": [256, 0, 256, 100, 7, 256, 0, 137],
    "tile": [257, 0, 255, 100, 7, 256, 0, 137],
}


def _announce(name):
    print(f"\n[gpu case] {name}", flush=True)
    sys.stdout.flush()


def _table(sizes, k, seed):
    """A (T, k) routing table whose experts receive exactly `sizes` rows and
    no token names an expert twice."""
    ids = np.repeat(np.arange(len(sizes), dtype=np.int32), sizes)
    T = len(ids) // k
    assert T * k == len(ids) and max(sizes) < T
    idx = ids.reshape(k, T).T.copy()  # token t takes ids t, T + t, ...: no repeats
    rng = np.random.default_rng(seed)
    idx = idx[rng.permutation(T)]
    g = rng.random(idx.shape).astype(np.float32)
    return idx, g


@pytest.mark.parametrize("form", ["plain", "gather", "dy"])
@pytest.mark.parametrize("path", ["strip", "tile"])
def test_weight_gradient_paths(path, form):
    """dy: moe_combine_ffn_bwd_gather (the combine backward inside the FFN
    backward, dYp formed from dY and the gate weights in the kernels where no
    kernel reads it); its scratch dYp, poisoned first, stays unwritten on the
    strip path and holds moe_combine_bwd's bits on the tile path, and its
    gate gradient is moe_combine_bwd's (on the strip path, to rounding: it
    comes from the dSwiGLU GEMM there)."""
    gather = form != "plain"
    sizes = SIZES[path]
    E, k, d, I = len(sizes), 2, 320, 192
    idx, g = _table(sizes, k, 71)
    T = idx.shape[0]
    w = MI.small_workload(f"wgrad_{path}_T{T}_d{d}_E{E}_k{k}_I{I}", T, d, E, k, I, seed=73,
                          backward=True)
    _announce(f"{w.name} form={form}")
    a = MI.generate(w, parts=("x", "Wg", "Wu", "Wd", "dY"))
    dev = U.upload(w, a)
    s = U.shape_of(w)
    buf = LayerBuffers(s, training=True, gather=gather)
    t = buf.t
    t["topk_idx"].copy_(torch.from_numpy(idx))
    t["topk_w"].copy_(torch.from_numpy(g))
    x = dev["x"]
    B.moe_permute(s, t["topk_idx"], x, t["offsets"], t["perm"], t["inv"], t["xp"], t["ws_permute"])
    if gather:
        B.moe_grouped_ffn_fwd_gather(s, x, t["perm"], t["offsets"], dev["Wg"], dev["Wu"], dev["Wd"],
                                     t["h"], t["a"], t["yp"], t["ws_ffn_fwd"])
    else:
        B.moe_grouped_ffn_fwd(s, t["xp"], t["offsets"], dev["Wg"], dev["Wu"], dev["Wd"], t["h"],
                              t["a"], t["yp"], t["ws_ffn_fwd"])
    B.moe_combine_bwd(s, dev["dY"], t["yp"], t["inv"], t["topk_w"], t["dyp"], t["dtopk_w"])
    # the gradients' buffers start poisoned: every element must be written
    for name in ("dw_gate", "dw_up", "dw_down"):
        t[name].fill_(float("nan"))
    if form == "dy":
        dyp_ref, dg_ref = t["dyp"].clone(), t["dtopk_w"].clone()
        t["dyp"].fill_(float("nan"))
        t["dtopk_w"].fill_(float("nan"))
        B.moe_combine_ffn_bwd_gather(s, x, t["perm"], t["inv"], t["offsets"], t["topk_w"],
                                     dev["Wg"], dev["Wu"], dev["Wd"], t["h"], t["a"], t["yp"],
                                     dev["dY"], t["dyp"], t["dtopk_w"], t["dxp"], t["dw_gate"],
                                     t["dw_up"], t["dw_down"], t["ws_ffn_bwd"])
        torch.cuda.synchronize()
        R = sum(sizes)
        if path == "strip":  # the gate gradient from the dSwiGLU GEMM: to rounding
            assert torch.isnan(t["dyp"][:R].float()).all(), "dYp written on the strip path"
            U.check("dtopk_w", U.np64(t["dtopk_w"]), U.np64(dg_ref), U.TOL["bf16"])
        else:
            assert torch.equal(t["dtopk_w"], dg_ref), "dtopk_w differs from moe_combine_bwd's"
            assert torch.equal(t["dyp"][:R].view(torch.int16), dyp_ref[:R].view(torch.int16)), \
                "the scratch dYp differs from the combine backward's"
    elif gather:
        B.moe_grouped_ffn_bwd_gather(s, x, t["perm"], t["offsets"], dev["Wg"], dev["Wu"],
                                     dev["Wd"], t["h"], t["a"], t["dyp"], t["dxp"], t["dw_gate"],
                                     t["dw_up"], t["dw_down"], t["ws_ffn_bwd"])
    else:
        B.moe_grouped_ffn_bwd(s, t["xp"], t["offsets"], dev["Wg"], dev["Wu"], dev["Wd"], t["h"],
                              t["a"], t["dyp"], t["dxp"], t["dw_gate"], t["dw_up"], t["dw_down"],
                              t["ws_ffn_bwd"])
    torch.cuda.synchronize()

    g64 = g.astype(np.float64)
    p = O.permute(idx, a["x"], E, 0, E)
    assert list(p["counts"]) == sizes
    assert np.array_equal(t["offsets"].cpu().numpy(), p["offsets"]), "group offsets differ"
    f = O.expert_ffn_fwd(p["Xp"], p["offsets"], a["Wg"], a["Wu"], a["Wd"])
    dYp, _ = O.combine_bwd(a["dY"], f["Yp"], p["inv"], g64, T, k)
    fb = O.expert_ffn_bwd(p["Xp"], p["offsets"], a["Wg"], a["Wu"], a["Wd"], f["Hg"], f["Hu"],
                          f["A"], dYp)
    R = int(p["offsets"][-1])
    tol = U.TOL["bf16"]
    U.check("dxp", U.np64(t["dxp"][:R]), fb["dXp"], tol)
    for gname, oname in (("dw_gate", "dWg"), ("dw_up", "dWu"), ("dw_down", "dWd")):
        got = U.np64(t[gname])
        assert np.isfinite(got).all(), f"{gname}: elements left unwritten"
        for e in range(E):
            U.check(f"{gname}[{e}]", got[e], fb[oname][e], tol)
            if sizes[e] == 0:
                assert not got[e].any(), f"{gname}[{e}]: an expert with no rows is not zero"


@pytest.mark.parametrize("path", ["strip", "tile"])
def test_gemm_engine_rounding_bound(path):
    """The bf16 MFMA GEMMs element by element at the precision their storage
    allows, on their own inputs (no chain of earlier roundings in between):
    the gate/up forward's H = Xp [Wg | Wu], the down projection's Yp = A Wd
    and its weight gradient dWd = A^T dYp (strip or tile kernel), each
    recomputed in fp64 from the bf16 tensors the kernel read."""
    sizes = SIZES[path]
    E, k, d, I = len(sizes), 2, 320, 192
    idx, g = _table(sizes, k, 79)
    T = idx.shape[0]
    w = MI.small_workload(f"engine_{path}_T{T}_d{d}_E{E}_k{k}_I{I}", T, d, E, k, I, seed=83,
                          backward=True)
    _announce(w.name)
    a = MI.generate(w, parts=("x", "Wg", "Wu", "Wd", "dY"))
    dev = U.upload(w, a)
    s = U.shape_of(w)
    buf = LayerBuffers(s, training=True)
    t = buf.t
    t["topk_idx"].copy_(torch.from_numpy(idx))
    t["topk_w"].copy_(torch.from_numpy(g))
    B.moe_permute(s, t["topk_idx"], dev["x"], t["offsets"], t["perm"], t["inv"], t["xp"],
                  t["ws_permute"])
    B.moe_grouped_ffn_fwd(s, t["xp"], t["offsets"], dev["Wg"], dev["Wu"], dev["Wd"], t["h"], t["a"],
                          t["yp"], t["ws_ffn_fwd"])
    B.moe_combine_bwd(s, dev["dY"], t["yp"], t["inv"], t["topk_w"], t["dyp"], t["dtopk_w"])
    B.moe_grouped_ffn_bwd(s, t["xp"], t["offsets"], dev["Wg"], dev["Wu"], dev["Wd"], t["h"], t["a"],
                          t["dyp"], t["dxp"], t["dw_gate"], t["dw_up"], t["dw_down"], t["ws_ffn_bwd"])
    torch.cuda.synchronize()
    off = t["offsets"].cpu().numpy()
    xp, h, act, yp, dyp = (U.np64(t[n][:off[-1]]) for n in ("xp", "h", "a", "yp", "dyp"))
    wg, wu, wd = U.np64(dev["Wg"]), U.np64(dev["Wu"]), U.np64(dev["Wd"])
    dwd = U.np64(t["dw_down"])
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            U.check_rounding_bound(f"h[{e}]", h[r0:r1], xp[r0:r1],
                                   np.concatenate([wg[e], wu[e]], 1))
            U.check_rounding_bound(f"yp[{e}]", yp[r0:r1], act[r0:r1], wd[e])
        U.check_rounding_bound(f"dw_down[{e}]", dwd[e], act[r0:r1].T, dyp[r0:r1])


def test_gemm_engine_rounding_bound_full_size():
    """The same element-by-element bound at the Qwen3 balanced shape in the
    bench's gathered form (the strip kernel with its real row blocks and
    column parts): H and Yp of the forward and the down weight gradient, for
    four sampled experts (each expert's GEMMs are computed by its own
    workgroups, so a sample covers the kernels' tile and column-part logic)."""
    w = MI.WORKLOADS["qwen3_balanced_fwdbwd_T4096_d2048_E128_k8_I768"]
    _announce(w.name + " engine bound")
    a = MI.generate(w)
    s, buf = U.run_layer(w, U.upload(w, a), gather=True)
    t = buf.t
    off = t["offsets"].cpu().numpy()
    perm = t["perm"].cpu().numpy()
    x = a["x"]
    for e in (0, 41, 86, 127):
        r0, r1 = off[e], off[e + 1]
        xp = x[perm[r0:r1] // w.k]  # the rows the gathered kernels read
        h, act, yp, dyp = (U.np64(t[n][r0:r1]) for n in ("h", "a", "yp", "dyp"))
        U.check_rounding_bound(f"h[{e}]", h, xp, np.concatenate([a["Wg"][e], a["Wu"][e]], 1))
        U.check_rounding_bound(f"yp[{e}]", yp, act, a["Wd"][e])
        U.check_rounding_bound(f"dw_down[{e}]", U.np64(t["dw_down"][e]), act.T, dyp)


def test_dy_form_down_wgrad_rounding_bound():
    """The strip kernel's dY form of dWd = sum_p (g_p A[p])^T dY[t_p] element
    by element against the rounding bound of its own operands (A rows scaled
    by their gate weights and rounded to bf16, nearest even, as the kernel
    does; the rows of dY through the token table), on 256-row, empty and
    ragged groups and a partial last column tile."""
    sizes = SIZES["strip"]
    E, k, d, I = len(sizes), 2, 320, 192
    idx, g = _table(sizes, k, 89)
    T = idx.shape[0]
    w = MI.small_workload(f"dyform_T{T}_d{d}_E{E}_k{k}_I{I}", T, d, E, k, I, seed=97,
                          backward=True)
    _announce(w.name)
    a = MI.generate(w, parts=("x", "Wg", "Wu", "Wd", "dY"))
    dev = U.upload(w, a)
    s = U.shape_of(w)
    buf = LayerBuffers(s, training=True, dy_form=True)
    t = buf.t
    t["topk_idx"].copy_(torch.from_numpy(idx))
    t["topk_w"].copy_(torch.from_numpy(g))
    x = dev["x"]
    B.moe_permute(s, t["topk_idx"], x, t["offsets"], t["perm"], t["inv"], t["xp"], t["ws_permute"])
    B.moe_grouped_ffn_fwd_gather(s, x, t["perm"], t["offsets"], dev["Wg"], dev["Wu"], dev["Wd"],
                                 t["h"], t["a"], t["yp"], t["ws_ffn_fwd"])
    t["dw_down"].fill_(float("nan"))
    B.moe_combine_ffn_bwd_gather(s, x, t["perm"], t["inv"], t["offsets"], t["topk_w"], dev["Wg"],
                                 dev["Wu"], dev["Wd"], t["h"], t["a"], t["yp"], dev["dY"],
                                 t["dyp"], t["dtopk_w"], t["dxp"], t["dw_gate"], t["dw_up"],
                                 t["dw_down"], t["ws_ffn_bwd"])
    torch.cuda.synchronize()
    off = t["offsets"].cpu().numpy()
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        perm = t["perm"][r0:r1].long()
        gw = t["topk_w"].reshape(-1)[perm]
        a_s = (t["a"][r0:r1].float() * gw[:, None]).to(torch.bfloat16)
        U.check_rounding_bound(f"dw_down[{e}]", U.np64(t["dw_down"][e]), U.np64(a_s).T,
                               U.np64(dev["dY"][perm // k]))
