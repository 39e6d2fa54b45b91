"""Host logic of bench.py (no GPU): the one-GPU refusal, the counter summary that scales
rocprofv3 FETCH_SIZE / WRITE_SIZE by the calibration copy, and the staleness rule of the
committed traffic figures."""

import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _write_csv(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, grid, value in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                        "Counter_Value": value})


def test_counter_summary_scales_by_the_calibration_copy(tmp_path):
    b = _bench()
    known_kib = b.ROWS * b.COLS * 2 / 1024.0
    key = "tile_copy_16384x16384_f16"
    sub = b.TRAFFIC_KERNELS[key][0]
    # the calibration copy reads half of what it moves in FETCH_SIZE units and writes it all;
    # the kernel under test reads 1.25x and writes 1x the calibration's bytes, twice
    fetch_dir, write_dir = str(tmp_path / "f"), str(tmp_path / "w")
    _write_csv(fetch_dir, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", "131072", known_kib / 2),
                                         ("__amd_rocclr_copyBuffer", "512", 3.0),
                                         (f"void tg::{sub}(tg::CopyArgs, int)", "1", known_kib / 2 * 1.25),
                                         (f"void tg::{sub}(tg::CopyArgs, int)", "1", known_kib / 2 * 1.25)])
    _write_csv(write_dir, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", "131072", known_kib),
                                         (f"void tg::{sub}(tg::CopyArgs, int)", "1", known_kib),
                                         (f"void tg::{sub}(tg::CopyArgs, int)", "1", known_kib)])
    out = str(tmp_path / "traffic.json")
    res = b.summarize_counters(fetch_dir, write_dir, out)
    assert res["_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert res["_calibration"]["write_factor"] == pytest.approx(1.0)
    rec = res[key]
    assert rec["bytes_per_launch"] == round(2.25 * b.ROWS * b.COLS * 2)
    assert rec["algorithmic_bytes"] == 2 * b.ROWS * b.COLS * 2
    assert rec["sources_sha"] == b.kernel_sources_sha("copy")
    assert json.load(open(out)) == res
    # kernels absent from the counter runs get no record
    assert "gemm_direct_256x256_bf16_nn" not in res


def test_traffic_goes_null_when_the_sources_change(tmp_path, monkeypatch):
    b = _bench()
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel": "k", "sources": "copy", "sources_sha": b.kernel_sources_sha("copy"),
           "bytes_per_launch": 123}
    (prof / "traffic.json").write_text(json.dumps({"tile_copy_16384x16384_f16": rec}))
    sha = b.kernel_sources_sha("copy")
    monkeypatch.setattr(b, "kernel_sources_sha", lambda which: sha if which == "copy" else "")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.traffic_for("tile_copy_16384x16384_f16") == 123
    assert b.traffic_for("not_a_kernel") is None
    rec["sources_sha"] = "0" * 16
    (prof / "traffic.json").write_text(json.dumps({"tile_copy_16384x16384_f16": rec}))
    assert b.traffic_for("tile_copy_16384x16384_f16") is None

