"""Host logic of bench.py, without a GPU: the roofline record built from kernel
timings, the counter summary built from rocprofv3 CSV files, and the one-GPU
guard."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from causal_linear_attention_amd.workloads import HEADLINE, WORKLOADS, kernel_bytes, kernel_flops  # noqa: E402


def test_roofline_record_of_the_dominant_kernel():
    w = WORKLOADS[HEADLINE]
    steps = 4
    # {name: (total ms, launches)} as the library's kernel timer reports it
    prof = {"state": (0.46, 2 * steps), "scan_prefix": (0.19, 2 * steps), "fwd": (1.1, steps),
            "rowstat": (0.22, steps), "bwdq_gstate": (1.8, steps), "scan_grad": (0.2, steps),
            "bwdkv": (2.24, steps)}
    kernels, roof = bench.kernel_records(w, prof, steps, 32, 1)
    assert roof["kernel"] == "bwdkv"
    d = kernels["bwdkv"]
    assert d["ms_avg"] == pytest.approx(0.56)
    units = w.B * w.H * w.L  # one launch covers every row of every head
    assert d["bytes_per_launch"] == pytest.approx(kernel_bytes(w)["bwdkv"] * units)
    assert d["flop_per_launch"] == pytest.approx(kernel_flops(w, 32)["bwdkv"] * units)
    # the binding roof is the slower of the two at peak: HBM for this kernel
    t_hbm = d["bytes_per_launch"] / 8e12
    t_mfma = d["flop_per_launch"] / 2.5e15
    assert t_hbm > t_mfma and roof["bound"] == "hbm" and roof["unit"] == "GB/s"
    assert roof["achieved"] == pytest.approx(d["bytes_per_launch"] / 0.56e-3 / 1e9, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 8000.0, rel=1e-3)
    # the state kernel and the prefix scan run in both passes: their launches each cover
    # all rows too (one window)
    assert kernels["state"]["bytes_per_launch"] == pytest.approx(kernel_bytes(w)["state"] * units)
    assert kernels["scan_prefix"]["bytes_per_launch"] == pytest.approx(kernel_bytes(w)["scan_prefix"] * units)
    assert kernels["scan_prefix"]["launches_per_step"] == 2


def test_units_per_launch_with_several_windows():
    # four windows: each launch of a chunk or scan kernel covers a quarter of the rows;
    # the dW pass's window count comes from its row contraction's launches
    w = WORKLOADS[HEADLINE]
    steps = 2
    prof = {"state": (1.0, 3 * 4 * steps), "scan_sum": (0.1, 4 * steps), "scan_window": (0.1, 4 * steps),
            "fwd": (1.0, 4 * steps), "bwdkv_dw": (2.0, 2 * steps), "dw": (0.5, 2 * steps)}
    kernels, _ = bench.kernel_records(w, prof, steps, 32, 4)
    units = w.B * w.H * w.L
    assert kernels["fwd"]["bytes_per_launch"] == pytest.approx(kernel_bytes(w)["fwd"] * units / 4)
    assert kernels["state"]["bytes_per_launch"] == pytest.approx(kernel_bytes(w)["state"] * units / 4)
    assert kernels["bwdkv_dw"]["bytes_per_launch"] == pytest.approx(kernel_bytes(w)["bwdkv_dw"] * units / 2)


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(r)


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path):
    w = WORKLOADS[HEADLINE]
    kn = "void slim::bwdkv_kernel<slim::KCfg<__bf16, 64, 256, 0, 32, 0, 0>, false>(slim::ChunkArgs)"
    qn = "void slim::bwdq_kernel<slim::KCfg<__bf16, 64, 256, 0, 32, 32, 32>, false>(slim::ChunkArgs)"
    cp = "__amd_rocclr_copyBuffer"
    d = str(tmp_path)
    # the calibration copy of 1 GiB reads FETCH_SIZE = 512 MiB and WRITE_SIZE = 1 GiB (KiB units)
    _counter_csv(os.path.join(d, "CF", "run_counter_collection.csv"),
                 [{"Kernel_Name": cp, "Counter_Name": "FETCH_SIZE", "Counter_Value": 524288}])
    _counter_csv(os.path.join(d, "CW", "run_counter_collection.csv"),
                 [{"Kernel_Name": cp, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1048576}])
    _counter_csv(os.path.join(d, "F", "run_counter_collection.csv"),
                 [{"Kernel_Name": kn, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000},
                  {"Kernel_Name": kn, "Counter_Name": "FETCH_SIZE", "Counter_Value": 3000},
                  {"Kernel_Name": qn, "Counter_Name": "FETCH_SIZE", "Counter_Value": 500}])
    _counter_csv(os.path.join(d, "W", "run_counter_collection.csv"),
                 [{"Kernel_Name": kn, "Counter_Name": "WRITE_SIZE", "Counter_Value": 100},
                  {"Kernel_Name": kn, "Counter_Name": "WRITE_SIZE", "Counter_Value": 300},
                  {"Kernel_Name": qn, "Counter_Name": "WRITE_SIZE", "Counter_Value": 50}])
    rec = bench.pmc_summary(d, w, 1 << 30)
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    k = rec["kernels"]["bwdkv"]
    assert k["dispatches"] == 2
    assert k["fetch_bytes"] == 2000 * 1024 * 2 and k["write_bytes"] == 200 * 1024
    # no separate gradient-state kernel: the dQ kernel carries it
    assert "bwdq_gstate" in rec["kernels"] and "bwdq" not in rec["kernels"]
    assert rec["source_hash"] == bench.kernel_source_hash()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr and r.stdout == ""
