"""Host-side logic of bench.py (no GPU): the multi-GPU refusal, the algorithmic
byte and flop counts the roofline divides by, checked against the counts written
out from the workload shapes, and the counter table's keying."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, timeout=120)
    assert r.returncode == 2
    assert b"one GPU" in r.stderr
    assert r.stdout.strip() == b""


def test_scan_algorithmic_bytes_long_context():
    # B1 L131072 D2048 N16 bf16: x, delta, z, y 2 bytes per (b,t,d); B, C 2 bytes per
    # (b,t,n); A (D x N), bias and D (D each) fp32; the fp32 final state (B x D x N)
    cfg = workloads.CONFIGS["S4"]
    bld = 131072 * 2048
    expect = 4 * 2 * bld + 2 * 2 * 131072 * 16 + 4 * (2048 * 16 + 2 * 2048) + 4 * 2048 * 16
    assert expect == 2_156_150_784
    assert bench.scan_alg_bytes(cfg) == expect


def test_scan_algorithmic_bytes_fp32():
    cfg = workloads.CONFIGS["S1"]                     # B1 L256 D64 N16 fp32
    expect = 4 * 4 * 256 * 64 + 2 * 4 * 256 * 16 + 4 * (64 * 16 + 2 * 64) + 4 * 64 * 16
    assert bench.scan_alg_bytes(cfg) == expect


def test_ssd_algorithmic_flops():
    # B2 L8192 H64 P64 N128 chunk 256: 32 chunks; C B^T once per chunk (causal half),
    # the masked product per head (causal half), chunk states and the carried-state
    # readout per head (full)
    cfg = workloads.CONFIGS["S5"]
    b, nch, H, P, N, Q = 2, 32, 64, 64, 128, 256
    expect = b * nch * (Q * Q * N + H * (Q * Q * P + 2 * (2 * Q * N * P)))
    assert bench.ssd_alg_flops(cfg) == pytest.approx(expect, rel=1e-12)
    assert round(expect / 1e9, 1) == 52.1


def test_counter_table_is_keyed_by_source_hash():
    # every entry names a workload and a 16-hex-digit hash of the scan sources;
    # figures taken on other sources are never reported (traffic null)
    for (key, h), fig in bench.COUNTERS.items():
        assert key in workloads.CONFIGS
        assert len(h) == 16 and int(h, 16) >= 0
        assert fig["traffic"] > 0 and fig["valu"] > 0
    assert len(bench.scan_source_hash()) == 16
