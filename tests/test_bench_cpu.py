"""bench.py's host-side figures: the algorithmic bytes and FLOPs it divides
by the measured kernel times, checked against the per-workload figures worked
out from the path's definition (read bf16 o, write FP8 codes and fp32 scales;
weights + activations + scales + bf16 z; 2*T*G*R*D FLOPs), the published
MI355X peaks it uses, and its refusal of more than one GPU."""
from __future__ import annotations

import subprocess
import sys
from pathlib import Path

import pytest

import bench
import workloads as wl

ROOT = Path(__file__).resolve().parents[1]


@pytest.mark.parametrize("name,quant_mb,gemm_mb,gflop", [
    ("decode", 12.73, 73.55, 8.59),        # T=64: HBM-bound GEMM, AI ~117 FLOP/B
    ("prefill", 1629.6, 889.2, 1099.5),    # T=8192
    ("full", 814.8, 478.2, 549.8),         # T=4096 (wo_b counted on its own)
    ("pow2", 204.0, 137.4, 137.4),         # T=2048, 8 live groups
])
def test_algorithmic_figures(name, quant_mb, gemm_mb, gflop):
    w = wl.WORKLOADS[name]
    assert abs(bench.kernel_bytes_quant(w) / 1e6 - quant_mb) <= 0.01 * quant_mb / 10
    assert abs(bench.kernel_bytes_gemm(w) / 1e6 - gemm_mb) <= 0.01 * gemm_mb / 10
    assert abs(bench.kernel_flops_gemm(w) / 1e9 - gflop) <= 0.01 * gflop / 10


def test_decode_quant_bytes_by_hand():
    """12,730,880 = 64 tokens x (128 heads x (1024 B read + 512 B written)
    + 16 groups x 32 blocks x 4 B of scales + 8 B position + 256 B table row)."""
    w = wl.WORKLOADS["decode"]
    assert bench.kernel_bytes_quant(w) == 64 * (128 * 1536 + 16 * 32 * 4 + 8 + 256) == 12730880


def test_decode_gemm_is_below_the_ridge_and_prefill_above():
    ridge = bench.FP8_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)  # FLOP per byte
    for name, below in (("decode", True), ("prefill", False)):
        w = wl.WORKLOADS[name]
        ai = bench.kernel_flops_gemm(w) / bench.kernel_bytes_gemm(w)
        assert (ai < ridge) == below, (name, ai, ridge)


def test_peaks_are_the_published_ones():
    assert bench.HBM_PEAK_GBS == 8000.0
    assert bench.FP8_PEAK_TFLOPS == 5000.0
    assert bench.BF16_PEAK_TFLOPS == 2500.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_device_info_degrades_without_a_device():
    """On a host without a GPU the device query returns an empty record
    instead of raising; on a GPU it reports CUs, clock and implied peaks."""
    import bench
    info = bench.device_info()
    assert info == {} or (info["cus"] > 0 and info["fp8_peak_tflops"] == 2 * info["bf16_peak_tflops"])
