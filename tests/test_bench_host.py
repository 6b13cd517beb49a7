"""CPU-only checks of bench.py's host logic: the one-GPU contract, the
throughput and byte formulas, and the committed traffic summaries it reads."""
from __future__ import annotations

import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_tflops_and_bytes():
    # 2*M*N*K FLOP in one second
    assert bench.tflops(1000, 1000, 1000, 1.0) == pytest.approx(2e-3)
    M, N, K = 8192, 8192, 8192
    assert bench.algorithmic_bytes(M, N, K) == 2 * (M * K + N * K) + 2 * M * N
    assert bench.algorithmic_bytes(M, N, K, elem=1) == (M * K + N * K) + 2 * M * N
    assert bench.algorithmic_bytes(4, 4, 4, extra=10) == 2 * 32 + 32 + 10
    assert bench.PEAK_FP8_TFLOPS == pytest.approx(2 * bench.PEAK_FP16_TFLOPS)
    assert bench.PEAK_FP16_TFLOPS == pytest.approx(2516.58, abs=0.01)


def test_source_hash_ignores_comments_only():
    h = bench.kernel_source_hash("f16")
    assert len(h) == 16 and h == bench.kernel_source_hash("f16")
    assert set(bench.PATH_SOURCES) == {"f16", "f16_ws", "f16_ex", "f16_acc16", "bf16", "fp8",
                                       "fp8_cs"}
    for files in bench.PATH_SOURCES.values():
        for f in files:
            assert (bench.CSRC / f).exists(), f


@pytest.mark.parametrize("path,workload,M,N,K,elem", [
    ("f16", "square_8192", 8192, 8192, 8192, 2),
    ("fp8", "square_8192", 8192, 8192, 8192, 1),
    ("f16", "skinny_64x16384x8192", 64, 16384, 8192, 2),
])
def test_recorded_traffic_is_plausible(path, workload, M, N, K, elem):
    # None when the summary is missing or was taken on other kernel code;
    # otherwise at least the bytes the product must move.
    t = bench.recorded_traffic(path, workload)
    summary = bench.traffic_summary(path, workload)
    assert summary.exists()
    assert "rocprofv3 --pmc FETCH_SIZE" in summary.read_text()
    if t is not None:
        assert t >= 0.95 * bench.algorithmic_bytes(M, N, K, elem=elem)


def test_cpu_baseline_single_thread_leg():
    # the oracle leg on a small workload: all threads, then one thread, each
    # over the whole D (the small workloads' oracle timing)
    import oracle
    from dense_gemm_18_amd import workloads as wl
    w = wl.WORKLOADS["tile_128x128x64"]
    A, B = wl.random_inputs(w)
    r = bench.cpu_baseline(lambda r0, r1, t: oracle.gemm_nt_f16(A[r0:r1], B, threads=t),
                           w.M, w.N, w.K, budget_s=5.0, single_thread=True)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
    st = r["single_thread"]
    assert st["cores"] == 1 and st["value"] > 0 and st["sample"].startswith("128 full rows")
