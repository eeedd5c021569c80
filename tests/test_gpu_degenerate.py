"""GPU parity on the degenerate cases of the method, each against the CPU
oracle (every output, element by element, as in test_gpu_parity.py):

* one expert, k = 1 (fp32): the layer is a dense SwiGLU MLP with gate
  weight 1;
* all router logits equal (a zero router): every token takes experts
  0 .. k-1 by the lower-id tie rule, so two groups hold every token and the
  other experts are empty (their weight gradients exactly zero);
* a local expert range that no token is routed to: no routed rows at all,
  every output of the expert path is zero;
* a single token.

Each runs the plain, the gathered and the dY form of the FFN (the combine
backward inside the FFN backward).
"""
import sys

import numpy as np
import pytest

import moe_inputs as MI
import gpu_util as U

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "dense_E1_k1_f32":  # (bf16 layers need E a multiple of 8)
        w = MI.small_workload("dense_f32_T100_d128_E1_k1_I192", 100, 128, 1, 1, 192, dtype="f32",
                              seed=62, x_sigma=0.5)
        return w, MI.generate(w)
    if name == "all_ties_zero_router":
        w = MI.small_workload("ties_T300_d128_E8_k2_I128", 300, 128, 8, 2, 128, seed=63)
        a = MI.generate(w)
        a["Wr"] = np.zeros_like(a["Wr"])
        return w, a
    if name == "no_local_rows":
        w = MI.small_workload("nolocal_T200_d128_E16_k2_I128_loc8_16", 200, 128, 16, 2, 128,
                              bias_sigma=1.0, e_lo=8, e_hi=16, seed=64)
        a = MI.generate(w)
        a["b"] = np.where(np.arange(16) < 4, 50.0, 0.0).astype(np.float32)
        return w, a
    if name == "single_token":
        w = MI.small_workload("one_T1_d64_E8_k4_I64", 1, 64, 8, 4, 64, bias_sigma=1.0, seed=65)
        return w, MI.generate(w)
    raise KeyError(name)


CASES = ["dense_E1_k1_f32", "all_ties_zero_router", "no_local_rows", "single_token"]


@pytest.mark.parametrize("name", CASES)
def test_degenerate(name):
    w, a = _case(name)
    print(f"\n[gpu case] {w.name}", flush=True)
    sys.stdout.flush()
    f, bw = U.oracle_full(w, a)
    counts = f["counts"]
    if name == "all_ties_zero_router":
        assert (f["idx"] == np.arange(w.k)).all() and counts[:w.k].tolist() == [w.T] * w.k
    if name == "no_local_rows":
        assert int(f["offsets"][-1]) == 0 and not f["y"].any()
    dev = U.upload(w, a)
    for gather in (False, True):
        _, buf = U.run_layer(w, dev, gather=gather)
        errs = U.compare_full(w, a, buf, f, bw)
    print({k: f"{v:.2e}" for k, v in errs.items()})
    # the combine backward inside the FFN backward, from poisoned buffers
    _, buf = U.run_layer(w, dev, dy_form=True, poison=True)
    U.compare_full(w, a, buf, f, bw, check_dyp=False)
