"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the roofline
arithmetic, the algorithmic byte counts, the traffic profile's guard and the
K x N operand of the transposed-B control."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_by_hand():
    n = 8192
    assert bench.algorithmic_bytes("f16", n, n, n) == 536870912            # A, B fp16 + C fp32
    assert bench.algorithmic_bytes("i8", n, n, n) == 2 * n * n + 4 * n * n
    assert bench.algorithmic_bytes("i4", n, n, n) == n * n + 4 * n * n
    # W4A16 decode layer: X 8 KiB, packed weights 8 MiB, scales 256 KiB, Y 8 KiB
    assert bench.algorithmic_bytes("w4a16", 1, 4096, 4096) == 8667136
    assert bench.algorithmic_bytes("w4a16", 16, 4096, 4096) == 8912896
    assert bench.algorithmic_bytes("w4a16", 128, 4096, 4096) == 10747904
    # quantiser: read fp16 W, write packed codes and fp16 scales (G = 128)
    assert bench.algorithmic_bytes("quantize", 1, 4096, 4096) == 2 * 4096 * 4096 + 4096 * 2048 + 2 * 4096 * 32


def test_roofline_bound_and_fraction():
    # FP16 8192^3 in 1 ms: compute-bound, 1099.5 TFLOP/s of 2500
    r = bench.roofline("f16", 8192, 8192, 8192, 1e-3)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(1099.511627776, abs=1e-3)   # rounded to 3 decimals
    assert r["frac"] == pytest.approx(1099.511627776 / 2500, abs=1e-4)
    # INT8 takes the int8 peak and TOP/s
    r = bench.roofline("i8", 4096, 4096, 4096, 1e-3)
    assert r["bound"] == "mfma" and r["unit"] == "TOP/s" and r["peak"] == 5000.0
    # W4A16 decode is bound by HBM: bytes / time against 8 TB/s
    r = bench.roofline("w4a16", 1, 4096, 4096, 4e-6)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(8667136 / 4e-6 / 1e9, abs=1e-3)
    # W4A16 at M = 128 is on the compute side of the ridge
    assert bench.roofline("w4a16", 128, 4096, 4096, 2e-5)["bound"] == "mfma"


def test_traffic_profile_guard(tmp_path, monkeypatch):
    """The committed counter summary is used only while the tile kernel's
    source is the one it was taken on."""
    text = open(bench.TRAFFIC_PROFILE).read()
    t = bench.measured_traffic()
    assert t is not None and t > bench.algorithmic_bytes("f16", 8192, 8192, 8192)
    assert f"traffic_bytes_per_launch: {t:.0f}" in text
    # a profile taken on another source is ignored
    other = tmp_path / "traffic.md"
    other.write_text(text.replace(bench.source_sha256(bench.TILE_SOURCE), "0" * 64))
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(other))
    assert bench.measured_traffic() is None
    # and so is a missing one
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "absent.md"))
    assert bench.measured_traffic() is None


@pytest.mark.parametrize("prec,N,K", [("i8", 40, 64), ("f16", 24, 16), ("i4", 47, 64), ("i4", 64, 32)])
def test_transposed_b_operand_by_element(prec, N, K):
    """bench.transpose_b (the K x N operand of the transposed-B control) holds
    B[n][k] at row k, column n; for INT4 element n of row k is nibble n % 2
    of byte n / 2 (low nibble = even n), two's complement."""
    import numpy as np
    from precision_dense_gemm_tiled_amd import inputs
    _, B = inputs.gemm_problem(prec, 3, N, K, seed=N + K)
    bt = bench.transpose_b(prec, B, N, K)
    if prec != "i4":
        assert bt.shape == (K, N) and bt.flags["C_CONTIGUOUS"]
        for n in range(N):
            for k in range(K):
                assert bt[k, n] == B[n, k] or (np.isnan(bt[k, n]) and np.isnan(B[n, k]))
        return

    def nib(byte, hi):
        v = (int(byte) >> (4 * hi)) & 0xF
        return v - 16 if v >= 8 else v

    assert bt.shape == (K, (N + 1) // 2)
    for n in range(N):
        for k in range(K):
            assert nib(bt[k, n // 2], n % 2) == nib(B[n, k // 2], k % 2), (n, k)
    if N % 2:
        assert not np.any(bt[:, -1] >> 4)   # the padding nibble is zero


def test_w4a16_trace_guard(tmp_path, monkeypatch):
    """The committed W4A16 kernel-trace durations are used only while the
    weight-only kernel source is the one they were taken on."""
    t = bench.w4a16_kernel_trace()
    assert t is not None and set(t) == {1, 16, 128} and all(v > 0 for v in t.values())
    text = open(bench.W4A16_TRACE_PROFILE).read()
    other = tmp_path / "trace.md"
    other.write_text(text.replace(bench.source_sha256(bench.W4A16_SOURCE), "0" * 64))
    monkeypatch.setattr(bench, "W4A16_TRACE_PROFILE", str(other))
    assert bench.w4a16_kernel_trace() is None
    monkeypatch.setattr(bench, "W4A16_TRACE_PROFILE", str(tmp_path / "absent.md"))
    assert bench.w4a16_kernel_trace() is None
