"""Host logic of bench.py that needs no GPU: the one-GPU guard, the roofline
choice and the source-hash gate on counter-derived traffic."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_counts_per_token_head():
    # d = 128, chunk 64: 12 d^2 + 8 C d dense FLOP; q, k, v, O bf16 and three fp32 gates
    assert bench.FLOP_FWD == 262144
    assert bench.BYTES_FWD == 1036
    assert bench.BYTES_SCAN == 768 + 256 + 256 + 24
    assert bench.BYTES_PREP == 512 + 12 + 256 + 24


def test_roofline_takes_the_roof_reached_last():
    # an intensity below the bf16 ridge (312 FLOP/B) is HBM-bound, above it MFMA-bound
    r = bench.roofline_of("none", 100.0, flop=100e9, nbytes=1e9)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["frac"] - 1e9 / 100e-6 / 8e12) < 1e-12
    r = bench.roofline_of("none", 100.0, flop=400e9, nbytes=1e9)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["frac"] - 400e9 / 100e-6 / 2.5e15) < 1e-12
    assert r["traffic"] is None


def test_traffic_is_null_once_sources_change(monkeypatch):
    entry = dict(bench.TRAFFIC["chunk_scan_bf16_kernel"])
    entry["sha256"] = "0" * 64
    monkeypatch.setitem(bench.TRAFFIC, "chunk_scan_bf16_kernel", entry)
    assert bench.traffic_bytes("chunk_scan_bf16_kernel") is None
    entry = dict(entry, sha256=bench.sources_sha256(entry["sources"]))
    monkeypatch.setitem(bench.TRAFFIC, "chunk_scan_bf16_kernel", entry)
    want = entry["fetch_kib"] * 1024 * bench.FETCH_FACTOR + entry["write_kib"] * 1024
    assert bench.traffic_bytes("chunk_scan_bf16_kernel") == round(want)
