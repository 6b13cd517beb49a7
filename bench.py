"""Throughput of the fp16 NT GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of gemm_nt_f16 (the whole hot path) on the 8192 x 8192 x
8192 workload: A [M,K] and B [N,K] fp16 drawn uniform[-1,1] from fixed seeds,
fp32 accumulation, D [M,N] fp16, all resident in HBM before timing starts.
Throughput is TFLOPS = 2*M*N*K / t (page "构建 Tiled GEMM", section "GEMM").

Prints one JSON line with the metric, a roofline object for the GEMM kernel
(achieved TFLOP/s from HIP events on the launch stream, against the MI355X
dense fp16 MFMA peak) and a CPU baseline (the oracle, on a bounded sample of
the same workload, on this host's cores).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

# MI355X dense fp16 MFMA peak: 256 CUs x 4096 FLOP/clock/CU x 2.4 GHz
# (AMD's published 2.5 PFLOP/s dense fp16 figure).
PEAK_FP16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = [ROOT / "dense_gemm_18_amd" / "csrc" / "gemm_kernels.h",
                  ROOT / "dense_gemm_18_amd" / "csrc" / "gemm_nt_f16.hip"]
TRAFFIC_SUMMARY = ROOT / "profiles" / "gemm_nt_f16_square_8192_traffic.md"


def tflops(M: int, N: int, K: int, seconds: float) -> float:
    """TFLOPS = 2*M*N*K / (t * 1e12): one multiply-add counts two."""
    return 2.0 * M * N * K / (seconds * 1e12)


def algorithmic_bytes(M: int, N: int, K: int) -> float:
    """A and B read once, D written once, fp16."""
    return 2.0 * (M * K + N * K + M * N)


def kernel_source_hash() -> str:
    """Hash of the kernel source's code: comments and whitespace are dropped,
    so only a change to the code itself invalidates recorded counters."""
    text = "\n".join(p.read_text() for p in KERNEL_SOURCES)
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    if not TRAFFIC_SUMMARY.exists():
        return None
    text = TRAFFIC_SUMMARY.read_text()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not b or h.group(1) != kernel_source_hash():
        return None
    return float(b.group(1))


def cpu_baseline(A, B, M, N, K, budget_s: float = 12.0) -> dict:
    """The oracle (untuned) on whole rows of D until ~budget_s of CPU work."""
    import oracle
    threads = oracle.threads_available()
    chunk = 64
    rows = 0
    t0 = time.perf_counter()
    while rows < M and time.perf_counter() - t0 < budget_s:
        r1 = min(M, rows + chunk)
        oracle.gemm_nt_f16(A[rows:r1], B, threads=threads)
        rows = r1
    dt = time.perf_counter() - t0
    return {
        "value": tflops(rows, N, K, dt),
        "unit": "TFLOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{rows} full rows of D ({rows}x{N}x{K}, {rows * N * K:.3e} MACs) in {dt:.1f} s",
    }


def copy_calibration(torch, nbytes: int = 1 << 30, reps: int = 3) -> int:
    """A plain copy of known size: each launch reads and writes `nbytes`."""
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_calibration_bytes_per_launch": nbytes, "launches": reps}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    # ~0.1 s of warm-up brings the clock to its steady level under the power
    # limit (the first tens of milliseconds of load run slower); the timed
    # region then spans well over 0.2 s.
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None, help="workload name (default: the 8192^3 GEMM)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    ap.add_argument("--sustain", type=float, default=0.0,
                    help="only run the GEMM back to back for this many seconds (for sampling "
                         "clock and power with amd-smi); prints the achieved TFLOPS")
    ap.add_argument("--torch-context", action="store_true",
                    help="also time torch.nn.functional.linear on the same inputs (context only)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this GEMM path is "
              "single-GPU and has no multi-GPU mode.", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        return copy_calibration(torch)

    from dense_gemm_18_amd import binding
    from dense_gemm_18_amd import build as hip_build
    from dense_gemm_18_amd import workloads as wl

    if not binding.library_path().exists():
        hip_build.build()
    name = args.workload or wl.HEADLINE
    w = wl.WORKLOADS[name]
    M, N, K = w.M, w.N, w.K
    dev = torch.device("cuda:0")

    A, B = wl.random_inputs(w)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dD = torch.empty((M, N), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    pa, pb, pd = dA.data_ptr(), dB.data_ptr(), dD.data_ptr()

    def step():
        rc = binding.gemm_nt_f16(pa, pb, pd, M, N, K, sptr)
        if rc != binding.GEMM_OK:
            raise RuntimeError(binding.gemm_nt_f16_strerror(rc))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    if args.sustain > 0:
        calls, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.sustain:
            for _ in range(50):
                step()
            torch.cuda.synchronize(dev)
            calls += 50
        dt = time.perf_counter() - t0
        print(json.dumps({"sustain_s": round(dt, 2), "calls": calls,
                          "tflops": round(tflops(M, N, K, dt / calls), 1)}), flush=True)
        return 0

    # Timed region: exactly `steps` calls, synchronised on both sides.  Each
    # launch is bracketed by HIP events on the launch stream.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    kernel_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_kernel_s = sum(kernel_ms) / len(kernel_ms) / 1e3
    median_ms = sorted(kernel_ms)[len(kernel_ms) // 2]
    ms_per_step = wall / args.steps * 1e3

    value = tflops(M, N, K, wall / args.steps)
    achieved = tflops(M, N, K, avg_kernel_s)
    traffic = recorded_traffic() if name == wl.HEADLINE else None
    props = torch.cuda.get_device_properties(dev)
    out = {
        "metric": "fp16 GEMM TFLOPS (2MNK/t) at 8192^3; % of MI355X dense fp16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": name, "M": M, "N": N, "K": K,
            "A": f"{w.a_dist} fp16, seed {w.seeds[0]}", "B": f"{w.b_dist} fp16, seed {w.seeds[1]}",
            "accumulate": "fp32", "layout": "A MxK, B NxK (D = A B^T), row-major",
            "tile": list(binding.gemm_nt_f16_tile(M, N, K)[:3]),
        },
        "pct_of_peak": round(100.0 * value / PEAK_FP16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(PEAK_FP16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
            "traffic": traffic,
            "kernel_ms_avg": round(avg_kernel_s * 1e3, 5),
            "kernel_ms_median": round(median_ms, 5),
            "kernel_ms_min": round(min(kernel_ms), 5),
            "kernel_ms_max": round(max(kernel_ms), 5),
            "algorithmic_flops_per_launch": 2.0 * M * N * K,
            "algorithmic_bytes_per_launch": algorithmic_bytes(M, N, K),
            "hbm_gbs_at_algorithmic_bytes": round(algorithmic_bytes(M, N, K) / avg_kernel_s / 1e9, 1),
        },
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    if args.torch_context:
        ts = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        lin = torch.nn.functional.linear          # A @ B^T with B stored [N, K]
        for _ in range(args.warmup):
            lin(dA, dB)
        ts[0].record(stream)
        for _ in range(args.steps):
            lin(dA, dB)
        ts[1].record(stream)
        torch.cuda.synchronize(dev)
        out["context_torch_linear_tflops"] = round(
            tflops(M, N, K, ts[0].elapsed_time(ts[1]) / args.steps / 1e3), 2)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(A, B, M, N, K)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
