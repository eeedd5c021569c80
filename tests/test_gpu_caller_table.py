"""GPU parity with a routing table handed in by the caller rather than made
by the router: slots that repeat an expert an earlier slot of the same token
names, ids outside the local range and ids outside [0, E).  The grouped path
(Xp copied by the permute, Xp read from x through perm, that with the
combine fused into the down projection, and that with the combine backward
inside the FFN backward), forward and the backward of every step after the
router, against the oracle, which visits each of a token's experts once,
through the first slot naming it.

Also the gather and combine kernels with more slots than 16-byte chunks per
row (d = 64 bf16, k = 16), where the slot data broadcast from lanes j < k
must reach every chunk."""
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


def _announce(name):
    print(f"\n[gpu case] {name}", flush=True)
    sys.stdout.flush()


def _table(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-2, E + 3, size=(T, k)).astype(np.int32)
    idx[3] = [5] * k                      # one expert in every slot
    idx[4] = [0, 1, 2, 3][:k]             # nothing local when e_lo >= 4
    idx[5] = ([11, 4] * k)[:k]            # two experts, each repeated
    idx[6] = ([-1, 99, 7, 7] * k)[:k]     # foreign ids, then a repeat
    g = rng.random((T, k)).astype(np.float32)
    return idx, g


@pytest.mark.parametrize("form", ["plain", "gather", "fused", "dy"])
@pytest.mark.parametrize("dtype,e_lo,e_hi", [("bf16", 4, 12), ("f32", 4, 12), ("bf16", 0, 16)])
def test_caller_table_grouped_path(dtype, e_lo, e_hi, form):
    gather = form != "plain"
    T, d, E, k, I = 45, 128, 16, 4, 192
    w = MI.small_workload(f"table_{dtype}_{e_lo}_{e_hi}", T, d, E, k, I, dtype=dtype, e_lo=e_lo,
                          e_hi=e_hi, seed=41, backward=True)
    _announce(f"caller table {w.name} {form}")
    a = MI.generate(w, parts=("x", "Wg", "Wu", "Wd", "dY"))
    idx, g = _table(T, E, k, 43)
    dev = U.upload(w, a)
    s = U.shape_of(w)
    buf = LayerBuffers(s, training=True, gather=gather, fused=form == "fused")
    t = buf.t
    t["topk_idx"].copy_(torch.from_numpy(idx))
    t["topk_w"].copy_(torch.from_numpy(g))
    x = dev["x"]
    B.moe_permute(s, t["topk_idx"], x, t["offsets"], t["perm"], t["inv"], t["xp"], t["ws_permute"])
    if form == "fused":
        B.moe_grouped_ffn_fwd_fused(s, x, t["perm"], t["inv"], t["topk_w"], t["offsets"],
                                    dev["Wg"], dev["Wu"], dev["Wd"], t["h"], t["a"], t["yp"],
                                    t["y"], t["ws_ffn_fwd_fused"])
    else:
        if gather:
            B.moe_grouped_ffn_fwd_gather(s, x, t["perm"], t["offsets"], dev["Wg"], dev["Wu"],
                                         dev["Wd"], t["h"], t["a"], t["yp"], t["ws_ffn_fwd"])
        else:
            B.moe_grouped_ffn_fwd(s, t["xp"], t["offsets"], dev["Wg"], dev["Wu"], dev["Wd"],
                                  t["h"], t["a"], t["yp"], t["ws_ffn_fwd"])
        B.moe_combine(s, t["yp"], t["inv"], t["topk_w"], t["y"])
    if form == "dy":  # the combine backward inside the FFN backward; dyp its scratch
        t["dyp"].fill_(float("nan"))
        B.moe_combine_ffn_bwd_gather(s, x, t["perm"], t["inv"], t["offsets"], t["topk_w"],
                                     dev["Wg"], dev["Wu"], dev["Wd"], t["h"], t["a"], t["yp"],
                                     dev["dY"], t["dyp"], t["dtopk_w"], t["dxp"], t["dw_gate"],
                                     t["dw_up"], t["dw_down"], t["ws_ffn_bwd"])
    elif gather:
        B.moe_combine_bwd(s, dev["dY"], t["yp"], t["inv"], t["topk_w"], t["dyp"], t["dtopk_w"])
        B.moe_grouped_ffn_bwd_gather(s, x, t["perm"], t["offsets"], dev["Wg"], dev["Wu"],
                                     dev["Wd"], t["h"], t["a"], t["dyp"], t["dxp"], t["dw_gate"],
                                     t["dw_up"], t["dw_down"], t["ws_ffn_bwd"])
    else:
        B.moe_combine_bwd(s, dev["dY"], t["yp"], t["inv"], t["topk_w"], t["dyp"], t["dtopk_w"])
        B.moe_grouped_ffn_bwd(s, t["xp"], t["offsets"], dev["Wg"], dev["Wu"], dev["Wd"], t["h"],
                              t["a"], t["dyp"], t["dxp"], t["dw_gate"], t["dw_up"], t["dw_down"],
                              t["ws_ffn_bwd"])
    B.moe_permute_bwd(s, t["dxp"], t["inv"], t["dx"])
    torch.cuda.synchronize()

    g64 = g.astype(np.float64)
    p = O.permute(idx, a["x"], E, e_lo, e_hi)
    f = O.expert_ffn_fwd(p["Xp"], p["offsets"], a["Wg"], a["Wu"], a["Wd"])
    y = O.combine(f["Yp"], p["inv"], g64, T, k)
    dYp, dG = O.combine_bwd(a["dY"], f["Yp"], p["inv"], g64, T, k)
    fb = O.expert_ffn_bwd(p["Xp"], p["offsets"], a["Wg"], a["Wu"], a["Wd"], f["Hg"], f["Hu"],
                          f["A"], dYp)
    dX = O.permute_bwd(fb["dXp"], p["inv"], T, k)

    R = int(p["offsets"][-1])
    assert (p["inv"].reshape(T, k)[3, 1:] == -1).all()  # the table does hold repeats
    assert np.array_equal(t["offsets"].cpu().numpy(), p["offsets"]), "group offsets differ"
    assert np.array_equal(t["perm"][:R].cpu().numpy(), p["perm"]), "perm differs"
    assert np.array_equal(t["inv"].cpu().numpy(), p["inv"]), "inv differs"
    if t["xp"] is not None:
        assert np.array_equal(U.np64(t["xp"][:R]), p["Xp"]), "xp is not an exact copy"
    tol = U.TOL[dtype]
    U.check("h", U.np64(t["h"][:R]), np.concatenate([f["Hg"], f["Hu"]], 1), tol)
    U.check("a", U.np64(t["a"][:R]), f["A"], tol)
    U.check("yp", U.np64(t["yp"][:R]), f["Yp"], tol)
    U.check("y", U.np64(t["y"]), y, tol)
    if form != "dy" or dtype == "f32":  # (bf16 dY form: dyp is not written here)
        U.check("dyp", U.np64(t["dyp"][:R]), dYp, tol)
    U.check("dtopk_w", U.np64(t["dtopk_w"]), dG, tol)
    assert not t["dtopk_w"].cpu().numpy()[p["inv"].reshape(T, k) < 0].any(), \
        "a dropped slot has a nonzero gate gradient"
    U.check("dxp", U.np64(t["dxp"][:R]), fb["dXp"], tol)
    for gname, oname in (("dw_gate", "dWg"), ("dw_up", "dWu"), ("dw_down", "dWd")):
        got = U.np64(t[gname])
        for e in range(e_hi - e_lo):
            U.check(f"{gname}[{e}]", got[e], fb[oname][e], tol)
            if p["counts"][e] == 0:
                assert not got[e].any()
    U.check("dx", U.np64(t["dx"]), dX, tol)


# more slots per token than 16-byte chunks per row: d = 64 bf16 is 8 chunks
WIDE_K = MI.small_workload("d64_k16_T100_d64_E32_k16_I64", 100, 64, 32, 16, 64, bias_sigma=1.0,
                           seed=47)


@pytest.mark.parametrize("gather", [False, True], ids=["plain", "gather"])
def test_more_slots_than_row_chunks(gather):
    w = WIDE_K
    _announce(f"{w.name} gather={gather}")
    a = MI.generate(w)
    f, bw = U.oracle_full(w, a)
    srt = -np.sort(-f["logits"], axis=1)
    assert (srt[:, w.k - 1] - srt[:, w.k]).min() > 1e-4, "seed gives a near-tie"
    _, buf = U.run_layer(w, U.upload(w, a), gather=gather)
    errs = U.compare_full(w, a, buf, f, bw)
    print({k: f"{v:.2e}" for k, v in errs.items()})
