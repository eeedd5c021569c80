"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
work per GEMM launch behind the roofline, and the HBM-counter summary."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_work_at_the_qwen3_shape():
    R, d, I, El, T = 32768, 2048, 768, 128, 4096
    gf = {n: f(R, d, I, El, T) / 1e9 for n, (f, _) in bench.GEMMS.items()}
    mb = {n: b(R, d, I, El, T) / 1e6 for n, (_, b) in bench.GEMMS.items()}
    # 4 R d I flops for the gate/up pair, 2 R d I for the down projection
    for n in ("ffn_gateup_fwd", "ffn_gateup_fwd_gather", "ffn_gateup_dgrad", "ffn_gateup_wgrad",
              "ffn_gateup_wgrad_gather"):
        assert gf[n] == pytest.approx(206.158, abs=1e-3)
    for n in ("ffn_down_fwd", "ffn_down_dgrad", "ffn_down_wgrad"):
        assert gf[n] == pytest.approx(103.079, abs=1e-3)
    # bytes: the expert weights (805 MB gate/up, 403 MB down) plus each
    # activation operand and result once
    assert mb["ffn_down_fwd"] == pytest.approx(402.65 + 50.33 + 134.22, abs=0.01)
    assert mb["ffn_down_wgrad"] == pytest.approx(mb["ffn_down_fwd"])
    assert mb["ffn_gateup_fwd"] == pytest.approx(134.22 + 805.31 + 100.66 + 50.33, abs=0.01)
    # the gathered forms read x (T rows) instead of Xp (R rows)
    assert mb["ffn_gateup_fwd"] - mb["ffn_gateup_fwd_gather"] == pytest.approx(2 * (R - T) * d / 1e6)
    assert mb["ffn_gateup_wgrad"] - mb["ffn_gateup_wgrad_gather"] == pytest.approx(2 * (R - T) * d / 1e6)
    assert mb["ffn_down_dgrad"] == pytest.approx(134.22 + 402.65 + 2 * 100.66, abs=0.01)


def test_counter_summary_scales_by_the_calibration_kernels(tmp_path):
    gemm9 = "void moe::gemm_bf16_kernel<256, 256, 2, 4, 2, 0, 0, 1, 1, 3, 9>(moe::GemmParams)"
    other = "void moe::gather_sum_kernel<unsigned short>(...)"
    rows_f = [("void at::native::reduce_kernel<...>", 512 * 1024),  # 1 GiB read counts half
              (gemm9, 1000.0), (gemm9, 3000.0), (other, 10.0)]
    rows_w = [("void at::native::FillFunctor<float>", 1024 * 1024),  # 1 GiB written counts once
              (gemm9, 200.0), (gemm9, 400.0), (other, 5.0)]

    def write(path, counter, rows):
        with open(path, "w", newline="") as fh:
            wr = csv.DictWriter(fh, ["Kernel_Name", "Counter_Name", "Counter_Value"])
            wr.writeheader()
            for k, v in rows:
                wr.writerow({"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})

    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    write(f, "FETCH_SIZE", rows_f)
    write(w, "WRITE_SIZE", rows_w)
    res = bench.summarize_pmc(str(f), str(w), 1024)
    assert res["calibration"]["read_factor"] == 2.0 and res["calibration"]["write_factor"] == 1.0
    k = res["kernels"]["ffn_gateup_fwd_gather"]  # role 9, averaged over its two dispatches
    assert k["read_bytes"] == 2000 * 1024 * 2 and k["write_bytes"] == 300 * 1024
    assert k["bytes_per_launch"] == k["read_bytes"] + k["write_bytes"]
    assert set(res["kernels"]) == {"ffn_gateup_fwd_gather"}
    assert res["source_hash"] == bench.kernel_source_hash()
