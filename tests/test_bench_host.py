"""Host logic of bench.py that needs no GPU: the profiler summaries."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from block_quantized_weight_02_amd import inputs  # noqa: E402


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_kernel_name_and_grid_of_plans():
    w = inputs.WORKLOADS["batch16_k4096_n14336"]
    p = {"kernel": 6, "rows": 16, "split_k": 1, "waves": 16, "kslices": 2}
    assert bench.kernel_name(p, w) == "gemv_tile16_kernel<0, 16, false, true, 1>"
    p32 = {"kernel": 6, "rows": 32, "split_k": 1, "waves": 8, "kslices": 1}
    assert bench.kernel_name(p32, w) == "gemv_tile16_kernel<0, 8, false, false, 2>"
    assert bench.plan_grid(p, w) == f"{224 * 64 * 16}x1x1"
    w5 = inputs.WORKLOADS["q8act_m32_k5120_n40"]
    p5 = {"kernel": 5, "rows": 32, "split_k": 4, "waves": 16, "kslices": 1}
    assert bench.kernel_name(p5, w5) == "gemv_mfma32w_kernel<16, false, 1>"
    assert bench.plan_grid(p5, w5) == "1024x4x1"
    w5b = inputs.WORKLOADS["q8act_m32_k5120_n32000"]
    p5b = {"kernel": 5, "rows": 32, "split_k": 1, "waves": 8, "kslices": 2}
    assert bench.kernel_name(p5b, w5b) == "gemv_mfma32w_kernel<8, false, 2>"
    assert bench.plan_grid(p5b, w5b) == f"{250 * 512}x1x1"


def test_summarize_pmc(tmp_path, capsys):
    K = "void q8::(anonymous namespace)::gemv_valu_kernel<1, 0, false, 8, false, false>(...)"
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    # the product (most dispatches), another gemv launch, and the quantize
    _write(tmp_path / "f.csv", hdr, [[K, 114688, "FETCH_SIZE", 1000.0]] * 3 + [[K, 8192, "FETCH_SIZE", 7.0],
           ["q8::quantize_act_kernel", 64, "FETCH_SIZE", 9.0]])
    _write(tmp_path / "w.csv", hdr, [[K, 114688, "WRITE_SIZE", 56.0]] * 3)
    _write(tmp_path / "cf.csv", hdr, [["__amd_rocclr_copyBuffer", 1, "FETCH_SIZE", 131072.0]] * 5)
    _write(tmp_path / "cw.csv", hdr, [["__amd_rocclr_copyBuffer", 1, "WRITE_SIZE", 262144.0]] * 5)
    bench.summarize_pmc("decode_k4096_n14336", *(str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv")))
    rec = json.loads(capsys.readouterr().out)
    assert rec["dispatches"]["gemv"] == 3
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    assert rec["traffic_read_bytes_per_launch"] == pytest.approx(1000.0 * 1024 * 2)
    assert rec["traffic_write_bytes_per_launch"] == pytest.approx(56.0 * 1024)
    assert rec["algorithmic_bytes_per_launch"] == 66125824
    assert rec["csrc_hash"] == bench.csrc_hash()


def test_summarize_kernel_trace_labels_configs(tmp_path, capsys):
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
           "Grid_Size_Z", "Workgroup_Size_X"]
    k0 = "void q8::(anonymous namespace)::gemv_valu_kernel<1, 0, false, 8, false, false>(...)"
    k6 = "void q8::(anonymous namespace)::gemv_tile16_kernel<0, 16, false, true, 1>(...)"
    rows = [[k0, 0, 11000 + i, 224 * 512, 1, 1, 512] for i in range(10)]
    rows += [[k0, 0, 3000, 16 * 512, 1, 1, 512] for _ in range(4)]
    rows += [[k6, 0, 14000, 224 * 1024, 1, 1, 1024] for _ in range(6)]
    _write(tmp_path / "t.csv", hdr, rows)
    line = {"metric": "m", "config": {"workload": "decode_k4096_n14336",
                                      "plan": {"kernel": 0, "rows": 1, "split_k": 1, "waves": 8, "kslices": 1}},
            "by_config": {
                "C1": {"workload": "decode_k1024_n1024",
                       "plan": {"kernel": 0, "rows": 1, "split_k": 1, "waves": 8, "kslices": 1}},
                "C4": {"workload": "batch16_k4096_n14336",
                       "plan": {"kernel": 6, "rows": 16, "split_k": 1, "waves": 16, "kslices": 2}}}}
    (tmp_path / "b.json").write_text("[bench] noise\n" + json.dumps(line) + "\n")
    bench.summarize_kernel_trace(str(tmp_path / "t.csv"), str(tmp_path / "b.json"))
    out = json.loads(capsys.readouterr().out)
    by = {tuple(k["configs"]): k for k in out["kernels"]}
    assert by[("T",)]["dispatches"] == 10
    assert by[("T",)]["median_us"] == pytest.approx(11.0045)
    assert by[("C1",)]["mean_us"] == pytest.approx(3.0)
    assert by[("C4",)]["dispatches"] == 6


def test_gpus_above_one_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
