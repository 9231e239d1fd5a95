"""Host-side behaviour of bench.py that needs no GPU: the single-GPU guard and the
traffic record's staleness check."""

import hashlib
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single-GPU" in r.stderr and r.stdout == ""


def _record(root, sources, fetch, write):
    h = hashlib.sha256()
    for s in sources:
        h.update(open(os.path.join(root, s), "rb").read())
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    json.dump({"sources": sources, "sources_sha256": h.hexdigest(), "fetch_size_kib": fetch, "write_size_kib": write,
               "fetch_factor": 2.0, "write_factor": 1.0},
              open(os.path.join(root, "profiles", "gemm_fp8_contig_gate_up_traffic.json"), "w"))


def test_traffic_record_is_used_only_for_unchanged_sources(tmp_path):
    root = str(tmp_path)
    src = os.path.join(root, "k.hip")
    open(src, "w").write("kernel v1\n")
    _record(root, ["k.hip"], 1000, 10)
    assert bench.measured_traffic(root) == (1000 * 2.0 + 10 * 1.0) * 1024.0
    open(src, "w").write("kernel v2\n")              # the kernel changed after the counters were taken
    assert bench.measured_traffic(root) is None


def test_committed_traffic_record_names_existing_sources():
    rec = json.load(open(os.path.join(ROOT, "profiles", "gemm_fp8_contig_gate_up_traffic.json")))
    for s in rec["sources"]:
        assert os.path.exists(os.path.join(ROOT, s))
    assert rec["fetch_size_kib"] > 0 and rec["write_size_kib"] > 0


def test_roofline_bound_follows_intensity():
    # gate-up-like launch: 481 GFLOP over 1032 MB is 466 FLOP/B, below the FP8 ridge of 625
    r = bench.roofline_entry("k", 481.0e9, 1032.0e6, 341.32e-6, bench.PEAK_FP8_TFLOPS, "")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS
    assert abs(r["frac"] - 1032.0e6 / 341.32e-6 / 8e12) < 1e-4 and r["frac"] == r["hbm_frac"]
    assert abs(r["mfma_frac"] - 481.0e9 / 341.32e-6 / 5e15) < 1e-4
    assert r["ridge_flop_per_byte"] == 625.0
    # dense-like launch: 240.5 GFLOP over 93 MB is far above the ridge
    r = bench.roofline_entry("k", 240.5e9, 93.0e6, 119e-6, bench.PEAK_FP8_TFLOPS, "")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["frac"] == r["mfma_frac"]
