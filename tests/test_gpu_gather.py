"""GPU parity of the fused-dispatch path: the gate/up GEMM and its weight
gradient read the rows of Xp from x through perm (moe_grouped_ffn_fwd_gather /
moe_grouped_ffn_bwd_gather) and Xp is never written.  Every output must match
the CPU oracle to the same tolerance as the plain path and be bit-identical to
the plain path (same operands, same summation order)."""
import sys

import numpy as np
import pytest
import torch

import moe_inputs as MI
import gpu_util as U
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"\n[gpu case] gather {name}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_gather_matches_oracle_and_plain_path(w):
    _announce(w.name)
    a = MI.generate(w)
    f, bw = U.oracle_full(w, a)
    dev = U.upload(w, a)
    s, g = U.run_layer(w, dev, gather=True)
    assert g["xp"] is None
    errs = U.compare_full(w, a, g, f, bw)
    print({k: f"{v:.2e}" for k, v in errs.items()})
    _, p = U.run_layer(w, dev)
    U.assert_same_outputs(g, p, int(f["offsets"][-1]), w.gate == "balanced")


def test_gather_capacity_drop_and_unwritten_rows():
    w = MI.small_workload("cap_T256_d128_E8_k2_I128", 256, 128, 8, 2, 128, bias_sigma=1.0, seed=31)
    _announce(w.name)
    a = MI.generate(w)
    cap = 301
    f, bw = U.oracle_full(w, a, R_cap=cap)
    s, g = U.run_layer(w, U.upload(w, a), R_cap=cap, poison=True, gather=True)
    U.compare_full(w, a, g, f, bw)
    R = int(g["offsets"][-1].item())
    assert R == cap
    # perm past the routed rows is never written (and never read by the GEMMs)
    assert (g["perm"][R:] == -7).all()


def test_gather_deterministic():
    w = SMALL[2]
    _announce("determinism " + w.name)
    a = MI.generate(w)
    dev = U.upload(w, a)
    s, b1 = U.run_layer(w, dev, poison=True, gather=True)
    _, b2 = U.run_layer(w, dev, poison=True, gather=True)
    U.assert_same_outputs(b1, b2, int(b1["offsets"][-1].item()), w.gate == "balanced")


@pytest.mark.parametrize("name", ["qwen3_balanced_fwdbwd_T4096_d2048_E128_k8_I768",
                                  "qwen3_natural_fwd_T4096_d2048_E128_k8_I768"])
def test_full_size_gather_equals_plain(name):
    """At the benchmark shape (balanced gate) and under natural routing (40
    empty experts, groups up to ~3,250 rows), fwd+bwd: the gathered path
    writes the same bits as the plain path, which the parity tests check
    against the oracle."""
    w = MI.WORKLOADS[name]
    if not w.backward:
        w = MI.Workload(**{**w.__dict__, "name": w.name + "_bwd", "backward": True})
    _announce(w.name)
    a = MI.generate(w)
    dev = U.upload(w, a)
    s, g = U.run_layer(w, dev, gather=True)
    R = int(g["offsets"][-1].item())
    _, p = U.run_layer(w, dev)
    U.assert_same_outputs(g, p, R, w.gate == "balanced")
    del p
    # and a sampled check against the oracle directly
    U.compare_sampled(w, a, g, np.r_[0:4, 4092:4096], experts=[0, 127])
