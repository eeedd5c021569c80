"""GPU parity of moe_route for a few tokens (T <= 16), where its logits come
from the few-token kernel (one workgroup per 16 bytes of a router row walks
all of d) instead of the MFMA router: logits within the fp32 bound, routing
bit for bit where it is well posed, gate weights, against the oracle; fp32
shapes whose E is not a multiple of 4 take the MFMA path and are checked the
same way; and the kernel's result does not change from call to call."""
import sys

import numpy as np
import pytest
import torch

import moe_inputs as MI
import gpu_util as U
from mixture_experts_layer_50_amd import binding as B
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

CASES = [
    MI.small_workload("rf_T1_d2048_E128_k8", 1, 2048, 128, 8, 64, bias_sigma=1.5, seed=91),
    MI.small_workload("rf_T8_d2048_E128_k8", 8, 2048, 128, 8, 64, bias_sigma=1.5, seed=92),
    MI.small_workload("rf_T16_d2048_E128_k8", 16, 2048, 128, 8, 64, bias_sigma=1.5, seed=93),
    MI.small_workload("rf_T3_d4160_E64_k4", 3, 4160, 64, 4, 64, bias_sigma=1.0, seed=94),
    MI.small_workload("rf_T12_d128_E512_k32", 12, 128, 512, 32, 64, bias_sigma=2.0, seed=95),
    MI.small_workload("rf_T5_d192_E8_k2", 5, 192, 8, 2, 64, seed=96),
    MI.small_workload("rf_f32_T7_d320_E64_k3", 7, 320, 64, 3, 64, dtype="f32", bias_sigma=1.0,
                      seed=97, x_sigma=0.5),
    MI.small_workload("rf_f32_T16_d128_E71_k5", 16, 128, 71, 5, 64, dtype="f32", bias_sigma=1.0,
                      seed=98, x_sigma=0.5),
    MI.small_workload("rf_f32_T2_d64_E7_k3", 2, 64, 7, 3, 64, dtype="f32", seed=99, x_sigma=0.5),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_few_token_route(w):
    print(f"\n[gpu case] moe_route {w.name}", flush=True)
    sys.stdout.flush()
    a = MI.generate(w, parts=("x", "Wr", "b"))
    dev = U.upload(w, a)
    s = U.shape_of(w)
    T, E, k = w.T, w.E, w.k
    L, idx, g = O.route(a["x"], a["Wr"], a.get("b"), k, "softmax_topk")
    outs = []
    for _ in range(2):
        logits = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
        ti = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
        tw = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
        B.moe_route(s, dev["x"], dev["Wr"], dev.get("b"), logits, ti, tw)
        torch.cuda.synchronize()
        outs.append((logits, ti, tw))
    logits, ti, tw = outs[0]
    for x0, x1 in zip(outs[0], outs[1]):
        assert torch.equal(x0, x1), "a second call differs"
    U.check("logits", U.np64(logits), L, 1e-5)
    U.assert_routing_well_posed(U.np64(logits), L, k)
    assert np.array_equal(ti.cpu().numpy(), idx)
    U.check("topk_w", U.np64(tw), g, 1e-5)
