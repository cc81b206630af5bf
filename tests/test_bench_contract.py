"""bench.py's host-side contract (no GPU): the one-GPU rule and the counter
arithmetic that turns rocprofv3 FETCH_SIZE / WRITE_SIZE into HBM bytes."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


@pytest.mark.parametrize("kernel,path_kind,w", [("gateup_gemv_decode_kernel", "decode", "q8b32"),
                                                 ("gateup_mfma_kernel", "prefill", "bf16")])
def test_traffic_scaling(tmp_path, kernel, path_kind, w):
    """Each counter is scaled by the factor that makes it read the probe's
    known size on the last three copy dispatches; earlier copies (weight
    uploads) and other kernels are ignored."""
    import bench
    mib = 64
    kib = mib * 1024
    name = "void moe::%s<2, 1, 1, 1>(moe::FfnArgs)" % kernel if path_kind == "decode" \
        else "moe::%s<128>(moe::FfnArgs)" % kernel
    # fetch reads half (factor 2), write reads exactly (factor 1)
    fetch_rows = [("__amd_rocclr_copyBuffer", 999999.0), (name, 1000.0), ("moe::other_kernel(x)", 5.0),
                  (name, 1200.0)] + [("__amd_rocclr_copyBuffer", kib / 2)] * 3
    write_rows = [("__amd_rocclr_copyBuffer", 1.0), (name, 10.0), (name, 30.0)] + \
                 [("__amd_rocclr_copyBuffer", float(kib))] * 3
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fcsv, "FETCH_SIZE", fetch_rows)
    _counter_csv(wcsv, "WRITE_SIZE", write_rows)
    out = tmp_path / "traffic.json"
    bench.record_traffic("wl", path_kind, w, str(fcsv), str(wcsv), mib << 20, rec_path=str(out))
    rec = json.load(open(out))["wl"]
    assert rec["kernel"] == kernel
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == pytest.approx(1100.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == pytest.approx(20.0 * 1024)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(1100.0 * 2048 + 20.0 * 1024)
    assert rec["fetch_launches"] == 2
