"""GPU parity of the combine backward run inside the gathered FFN backward
(moe_combine_ffn_bwd_gather): dYp is written (as scratch) only when a kernel
reads it -- the bf16 tile kernels, when an expert has more than 256 rows, and
the fp32 path -- and otherwise the rows g * dY[t] of dYp are formed inside
the kernels from dY and the gate weights, and the gate gradient comes from
the dSwiGLU GEMM.  Every output must match the oracle to the same tolerance
as the other forms; the forward and its outputs (routing, H, A, Yp, y) must
be the gathered form's bits, and on the tile path (and in fp32) so must every
output.  Runs start from poisoned buffers, dYp included, so a kernel that
read the scratch unwritten would show NaN."""
import sys

import numpy as np
import pytest
import torch

import moe_inputs as MI
import gpu_util as U
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

SAME_BITS = ("logits", "topk_idx", "topk_w", "offsets", "perm", "inv", "h", "a", "yp", "y")


def _announce(name):
    print(f"\n[gpu case] dy form {name}", flush=True)
    sys.stdout.flush()


def _same_bits_as_gather(d, g, R, balanced):
    for name in SAME_BITS:
        t1, t2 = d.t.get(name), g.t.get(name)
        if t1 is None or t2 is None or (balanced and name == "logits"):
            continue
        if name in ("perm", "h", "a", "yp"):
            t1, t2 = t1[:R], t2[:R]
        v1 = t1 if t1.dtype == torch.int32 else t1.view(torch.uint8)
        v2 = t2 if t2.dtype == torch.int32 else t2.view(torch.uint8)
        assert torch.equal(v1, v2), f"{name} differs from the gathered form"


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_dy_form_matches_oracle(w):
    _announce(w.name)
    a = MI.generate(w)
    f, bw = U.oracle_full(w, a)
    dev = U.upload(w, a)
    s, d = U.run_layer(w, dev, poison=True, dy_form=True)
    errs = U.compare_full(w, a, d, f, bw, check_dyp=False)
    print({k: f"{v:.2e}" for k, v in errs.items()})
    _, g = U.run_layer(w, dev, gather=True)
    R = int(f["offsets"][-1])
    _same_bits_as_gather(d, g, R, w.gate == "balanced")
    if w.dtype == "f32" or np.diff(f["offsets"]).max() > 256:  # dYp written and read as is
        U.assert_same_outputs(d, g, R, w.gate == "balanced")


def test_dy_form_capacity_drop():
    """Dropped slots (R_cap < T*k): they get no dYp row and a zero gate
    gradient; the kept rows' tokens and gate weights come from perm."""
    w = MI.small_workload("cap_T256_d128_E8_k2_I128", 256, 128, 8, 2, 128, bias_sigma=1.0, seed=31)
    _announce(w.name)
    a = MI.generate(w)
    cap = 301
    f, bw = U.oracle_full(w, a, R_cap=cap)
    s, d = U.run_layer(w, U.upload(w, a), R_cap=cap, poison=True, dy_form=True)
    U.compare_full(w, a, d, f, bw, check_dyp=False)
    assert int(d["offsets"][-1].item()) == cap


def test_dy_form_deterministic():
    w = SMALL[2]
    _announce("determinism " + w.name)
    a = MI.generate(w)
    dev = U.upload(w, a)
    s, b1 = U.run_layer(w, dev, poison=True, dy_form=True)
    _, b2 = U.run_layer(w, dev, poison=True, dy_form=True)
    R = int(b1["offsets"][-1].item())
    for name, t1 in b1.t.items():
        if t1 is None or name.startswith("ws_") or name in ("dyp", "xp") or \
                (w.gate == "balanced" and name == "logits"):
            continue
        t2 = b2.t[name]
        if name in ("perm", "h", "a", "yp", "dxp"):
            t1, t2 = t1[:R], t2[:R]
        v1 = t1 if t1.dtype == torch.int32 else t1.view(torch.uint8)
        v2 = t2 if t2.dtype == torch.int32 else t2.view(torch.uint8)
        assert torch.equal(v1, v2), f"{name} differs between two runs"


def _dy_down_wgrad_bound(name, buf, dy, k, e):
    """dWd[e] of the strip kernel's dY form against the rounding bound of its
    own operands: A rows scaled by their gate weights and rounded to bf16
    (round to nearest even, as the kernel does), and the rows of dY."""
    t = buf.t
    off = t["offsets"].cpu().numpy()
    r0, r1 = int(off[e]), int(off[e + 1])
    perm = t["perm"][r0:r1].long()
    gw = t["topk_w"].reshape(-1)[perm]
    a_s = (t["a"][r0:r1].float() * gw[:, None]).to(torch.bfloat16)
    U.check_rounding_bound(name, U.np64(t["dw_down"][e]), U.np64(a_s).T, U.np64(dy[perm // k]))


def test_full_size_balanced_dy_form():
    """The benchmark shape (every expert 256 rows: the strip kernel, dYp never
    written), sampled tokens and experts against the oracle, and the down
    weight gradient of four experts element by element against its rounding
    bound."""
    w = MI.WORKLOADS["qwen3_balanced_fwdbwd_T4096_d2048_E128_k8_I768"]
    _announce(w.name)
    a = MI.generate(w)
    dev = U.upload(w, a)
    s, d = U.run_layer(w, dev, poison=True, dy_form=True)
    U.compare_sampled(w, a, d, np.r_[0:8, 777, 3000:3004, 4095], experts=[0, 1, 63, 127],
                      check_dyp=False)
    R = int(d["offsets"][-1].item())
    assert torch.isnan(d["dyp"][:R].float()).all(), "dYp was written although no kernel reads it"
    for e in (0, 41, 86, 127):
        _dy_down_wgrad_bound(f"dw_down[{e}]", d, dev["dY"], w.k, e)


def test_full_size_natural_dy_form():
    """Natural routing at the Qwen3 shape (40 empty experts, groups up to
    ~3,250 rows: dYp written, the tile kernels and the dSwiGLU GEMM read it):
    every output the gathered form's bits, and sampled tokens, the largest,
    an empty and two ordinary experts against the oracle."""
    w = MI.WORKLOADS["qwen3_natural_fwd_T4096_d2048_E128_k8_I768"]
    w = MI.Workload(**{**w.__dict__, "name": w.name + "_bwd", "backward": True})
    _announce(w.name)
    a = MI.generate(w)
    dev = U.upload(w, a)
    s, d = U.run_layer(w, dev, poison=True, dy_form=True)
    counts = np.diff(d["offsets"].cpu().numpy())
    assert counts.min() == 0 and counts.max() > 1000
    _, g = U.run_layer(w, dev, gather=True)
    U.assert_same_outputs(d, g, int(d["offsets"][-1].item()))
    del g
    experts = [int(counts.argmax()), int(np.flatnonzero(counts == 0)[0]), 3, 100]
    U.compare_sampled(w, a, d, np.r_[0:8, 2048:2052, 4092:4096], experts=experts)


def test_full_size_dsv3_dy_form():
    """One rank's share of the DeepSeek-V3 shape (32 local experts of 1,024
    rows, R_cap = T*k = 262,144 rows of 7,168: dYp of 3.5 GiB, written and
    read from each tile's first row): every output the gathered form's bits
    (that form is checked against the oracle at this shape)."""
    w = MI.WORKLOADS["dsv3_ep8_rank_fwdbwd_T32768_d7168_E256_loc32_k8_I2048"]
    _announce(w.name)
    a = MI.generate(w)
    dev = U.upload(w, a)
    del a
    s, d = U.run_layer(w, dev, dy_form=True)
    R = int(d["offsets"][-1].item())
    assert R == 32768
    _, g = U.run_layer(w, dev, gather=True)
    U.assert_same_outputs(d, g, R, True)
