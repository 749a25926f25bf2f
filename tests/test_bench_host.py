"""Host-side logic of bench.py (no GPU): the operation count behind the roofline,
the traffic summary's calibration by the copy probe, the rule that drops the
traffic figure once the forward kernel's source has changed, and the refusal of
more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_operation_count():
    # 3 operations per state and step over 2^16 states x 256 steps, plus the
    # 2^16 - 2^(16-K) eliminations at each of 255 transitions, both passes,
    # plus the 2^16 - 1 comparisons of pass 1's final argmin
    n = 65536
    for K in (1, 2, 3, 4):
        per_pass = 256 * 3 * n + 255 * (n - n // 2 ** K)
        assert bench.ops_per_tile_encode(K) == 2 * per_pass + n - 1
    assert bench.ops_per_tile_encode(2) == 125_796_351


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                          "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_summary_is_calibrated_by_the_copy_probe(tmp_path):
    # the 1 MiB copy reads as 512 KiB of FETCH_SIZE (scale 2) and 1024 KiB of
    # WRITE_SIZE (scale 1); two pass-2 launches of 8 and 24 tiles, a pass-1 launch
    # of 8 tiles, split over two rows (counter dimensions) each
    fwd2 = "void exl3::(anonymous namespace)::viterbi_fwd_kernel<2, 2>(float const*)"
    fwd1 = "void exl3::(anonymous namespace)::viterbi_fwd_kernel<2, 1>(float const*)"
    copy = "__amd_rocclr_copyBuffer"

    def rows(counter, copy_kib, per_tile_kib):
        out = [{"Dispatch_Id": 1, "Kernel_Name": copy, "Grid_Size": 1 << 20,
                "Counter_Name": counter, "Counter_Value": copy_kib},
               {"Dispatch_Id": 2, "Kernel_Name": copy, "Grid_Size": 64,
                "Counter_Name": counter, "Counter_Value": 1.0}]
        for d, name, tiles in ((3, fwd2, 8), (4, fwd2, 24), (5, fwd1, 8)):
            for half in (0, 1):
                out.append({"Dispatch_Id": d, "Kernel_Name": name, "Grid_Size": tiles * 1024,
                            "Counter_Name": counter,
                            "Counter_Value": per_tile_kib[name] * tiles / 2})
        out.append({"Dispatch_Id": 9, "Kernel_Name": fwd2, "Grid_Size": 1024,
                    "Counter_Name": "OTHER", "Counter_Value": 1e9})
        return out

    f_csv, w_csv = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_csv(f_csv, rows("FETCH_SIZE", 512.0, {fwd2: 3.0, fwd1: 5.0}))
    _write_csv(w_csv, rows("WRITE_SIZE", 1024.0, {fwd2: 1000.0, fwd1: 500.0}))
    out = bench.summarize_traffic(str(f_csv), str(w_csv), 1, out_path=str(tmp_path / "t.json"))
    assert out["calibration"]["FETCH_SIZE"]["scale"] == 2.0
    assert out["calibration"]["WRITE_SIZE"]["scale"] == 1.0
    p2, p1 = out["per_launch"]["K2"]["pass2"], out["per_launch"]["K2"]["pass1"]
    assert p2["fetch_bytes_per_tile"] == 3.0 * 1024 * 2.0
    assert p2["write_bytes_per_tile"] == 1000.0 * 1024
    assert p1["fetch_bytes_per_tile"] == 5.0 * 1024 * 2.0
    assert out["source_sha256"] == bench.file_sha(bench.FWD_SOURCE)
    assert json.load(open(tmp_path / "t.json")) == out


def test_traffic_is_dropped_once_the_kernel_source_changes(tmp_path, monkeypatch):
    entry = {"pass1": {"fetch_bytes_per_tile": 1.0, "write_bytes_per_tile": 2.0}}
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    path.write_text(json.dumps({"source_sha256": bench.file_sha(bench.FWD_SOURCE),
                                "per_launch": {"K2": entry}}))
    assert bench.load_traffic(2) == entry
    path.write_text(json.dumps({"source_sha256": "0" * 64, "per_launch": {"K2": entry}}))
    assert bench.load_traffic(2) is None
    path.unlink()
    assert bench.load_traffic(2) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_roofline_rates_pass_two_of_the_final_encode(tmp_path, monkeypatch):
    # 8 pass-2 launches of 8,192 tiles in 80 ms: 8 x 8192 x ops / 0.08 s
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "none.json"))
    kern = {"fwd1": (70.0, 22, 8 * 8192 + 14 * 256), "fwd2": (80.0, 8, 8 * 8192),
            "fwd_cost": (5.0, 14, 14 * 256)}
    r = bench.roofline_line(2, kern, 380000.0, 1)
    ops = bench.ops_per_pass(2, False)
    assert ops == 256 * 3 * 65536 + 255 * (65536 - 16384) == 62_865_408
    assert r["achieved"] == round(8 * 8192 * ops / 0.08 / 1e12, 3)
    assert r["frac"] == round(r["achieved"] / bench.PEAK_FP32_TFLOPS, 4)
    assert r["avg_launch_ms"] == 10.0 and r["avg_tiles_per_launch"] == 8192.0
    assert r["traffic"] is None and "peak_issue" not in r
    whole = 380000.0 * bench.ops_per_tile_encode(2) / 1e12 / bench.PEAK_FP32_TFLOPS
    assert r["whole_path_frac"] == round(whole, 4)
