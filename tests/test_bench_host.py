"""Host-side logic of bench.py (no GPU): the one-GPU contract and the HBM
traffic bookkeeping (counter files -> bytes per launch, gated by a hash of
the kernel sources)."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
GRID_C2, GRID_C3 = 512 * 512, 2048 * 512


def _counter_dir(tmp_path, name, rows):
    d = tmp_path / name / "host"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, row in enumerate(rows):
            kernel, counter, value = row[:3]
            grid = row[3] if len(row) > 3 else 64
            w.writerow({"Dispatch_Id": i + 1, "Grid_Size": grid, "Kernel_Name": kernel,
                        "Counter_Name": counter, "Counter_Value": value})
    return str(tmp_path / name)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_scaled_by_copy_calibration_and_gated_by_source_hash(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    fwd = bench.TRAFFIC_KERNELS["attn_fwd_mfma_kernel"][0] + "(attn::FwdParams)"
    split = bench.TRAFFIC_KERNELS["paged_decode_split_kernel"][0] + " 2>(attn::DecodeParams)"
    comb = bench.TRAFFIC_KERNELS["paged_decode_combine_kernel"][0] + ", 128>(attn::DecodeParams)"
    copy = "__amd_rocclr_copyBuffer"
    # a 1 GiB copy whose fetch counter reads half the bytes (factor 2) and whose
    # write counter reads all of them (factor 1); two dispatches per kernel,
    # averaged
    cf = _counter_dir(tmp_path, "cf", [(copy, "FETCH_SIZE", 524288.0)] * 3)
    cw = _counter_dir(tmp_path, "cw", [(copy, "WRITE_SIZE", 1048576.0)] * 3)
    # the two prefills of the step are one kernel, told apart by their grids
    mf = _counter_dir(tmp_path, "mf", [(fwd, "FETCH_SIZE", 100.0, GRID_C2),
                                       (fwd, "FETCH_SIZE", 9000.0, GRID_C3),
                                       (fwd, "FETCH_SIZE", 300.0, GRID_C2),
                                       (split, "FETCH_SIZE", 1000.0), (comb, "FETCH_SIZE", 10.0)])
    mw = _counter_dir(tmp_path, "mw", [(fwd, "WRITE_SIZE", 50.0, GRID_C2),
                                       (fwd, "WRITE_SIZE", 700.0, GRID_C3),
                                       (fwd, "WRITE_SIZE", 50.0, GRID_C2),
                                       (split, "WRITE_SIZE", 4.0), (comb, "WRITE_SIZE", 1.0)])
    bench.write_traffic(mf, mw, cf, cw)
    t = json.loads(out.read_text())
    assert abs(t["fetch_factor"] - 2.0) < 1e-12 and abs(t["write_factor"] - 1.0) < 1e-12
    e = t["attn_fwd_mfma_kernel"]
    assert e["dispatches"] == [2, 2]
    assert e["fetch_bytes"] == 200 * 1024 * 2 and e["write_bytes"] == 50 * 1024
    assert e["bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"]
    assert t["paged_decode_split_kernel"]["bytes_per_launch"] == 1000 * 1024 * 2 + 4 * 1024
    el = t["attn_fwd_mfma_kernel_long"]
    assert el["dispatches"] == [1, 1]
    assert el["fetch_bytes"] == 9000 * 1024 * 2 and el["write_bytes"] == 700 * 1024
    # kernels of runs that were not given are left out
    assert "paged_decode_prefix_kernel" not in t and "attn_bwd_dkdv_kernel" not in t
    # reported only while the kernel sources are the ones measured
    assert bench.load_traffic("attn_fwd_mfma_kernel") == e["bytes_per_launch"]
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    assert bench.load_traffic("attn_fwd_mfma_kernel") is None

