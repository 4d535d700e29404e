"""Host logic of bench.py, on the CPU: the one-GPU refusal, the scaling of
rocprofv3 FETCH_SIZE / WRITE_SIZE counters by a plain copy of known size,
the per-dispatch counter means, and the rule that a traffic record is
reported only while its kernel's sources are the ones it was measured on."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(monkeypatch, root):
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    monkeypatch.setattr(b, "ROOT", str(root))
    return b


def _counter_csv(path, rows):
    """rows: (kernel, dispatch, counter, value KiB); one row per dispatch and
    counter instance."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, d, c, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr
    assert not r.stdout.strip()  # no JSON line


def test_counters_scaled_by_the_copy_and_checked_against_sources(tmp_path, monkeypatch):
    b = _bench(monkeypatch, tmp_path)
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "dynamic_quantized_gemm_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "k.hip").write_text("kernel source v1\n")
    copy = "__amd_rocclr_copyBuffer"
    # the 1 GiB copy reads as 655,360 KiB fetched (two instances summed in one
    # dispatch) and 2^20 KiB written: scales 1.6 and 1.0; a small copy of 4 KiB
    # is not a 1 GiB one and is left out
    _counter_csv(tmp_path / "cf.csv", [(copy, 1, "FETCH_SIZE", 327680.0), (copy, 1, "FETCH_SIZE", 327680.0),
                                       (copy, 2, "FETCH_SIZE", 655360.0), (copy, 3, "FETCH_SIZE", 4.0)])
    _counter_csv(tmp_path / "cw.csv", [(copy, 1, "WRITE_SIZE", 2 ** 20), (copy, 2, "WRITE_SIZE", 2 ** 20)])
    # the kernel: 1000 and 3000 KiB fetched (mean 2000), 500 KiB written
    _counter_csv(tmp_path / "kf.csv", [("k_x<1>(int)", 7, "FETCH_SIZE", 1000.0),
                                       ("k_x<1>(int)", 8, "FETCH_SIZE", 3000.0),
                                       ("k_other(int)", 9, "FETCH_SIZE", 99.0)])
    _counter_csv(tmp_path / "kw.csv", [("k_x<1>(int)", 7, "WRITE_SIZE", 500.0),
                                       ("k_x<1>(int)", 8, "WRITE_SIZE", 500.0)])
    b.write_counters(str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"),
                     [f"lab=k_x<1>={tmp_path / 'kf.csv'}={tmp_path / 'kw.csv'}=2048000=csrc/k.hip"])
    rec = json.loads((tmp_path / "profiles" / "traffic.json").read_text())["lab"]
    assert rec["dispatches"] == [2, 2]
    assert rec["fetch_scale"] == 1.6 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes"] == 3276800 and rec["write_bytes"] == 512000
    assert rec["traffic_over_algorithmic"] == round((3276800 + 512000) / 2048000, 3)
    assert b.traffic_record("lab")["bytes_per_launch"] == 3276800 + 512000
    (src / "k.hip").write_text("kernel source v2\n")  # the kernel changed since
    assert b.traffic_record("lab") is None
    assert b.traffic_record("missing") is None


def test_counter_means_per_dispatch(tmp_path, monkeypatch, capsys):
    b = _bench(monkeypatch, tmp_path)
    _counter_csv(tmp_path / "p.csv", [("k_gemm<2>(x)", 1, "SQ_BUSY_CYCLES", 10.0),
                                      ("k_gemm<2>(x)", 1, "SQ_BUSY_CYCLES", 30.0),
                                      ("k_gemm<2>(x)", 2, "SQ_BUSY_CYCLES", 60.0),
                                      ("k_gemm<2>(x)", 2, "GRBM_GUI_ACTIVE", 5.0),
                                      ("k_other(x)", 3, "SQ_BUSY_CYCLES", 1e9)])
    b.summarize_pmc(str(tmp_path / "p.csv"), "k_gemm<2>")
    out = json.loads(capsys.readouterr().out)
    assert out["SQ_BUSY_CYCLES"] == {"mean": 50.0, "dispatches": 2}
    assert out["GRBM_GUI_ACTIVE"] == {"mean": 5.0, "dispatches": 1}
    with pytest.raises(SystemExit):
        b._counter_means(str(tmp_path / "p.csv"), "FETCH_SIZE", "k_gemm")
