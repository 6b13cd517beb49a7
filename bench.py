"""Throughput of the NT GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--path f16|f16_ex|f16_ws|f16_acc16|bf16|fp8|fp8_cs]

A step is one call of the chosen entry point (the whole hot path): by
default gemm_nt_f16 on the 8192 x 8192 x 8192 workload, A [M,K] and B [N,K]
fp16 drawn uniform[-1,1] from fixed seeds, fp32 accumulation, D [M,N] fp16,
all resident in HBM before timing starts.  Throughput is
TFLOPS = 2*M*N*K / t (page "构建 Tiled GEMM", section "GEMM").

The other paths time the library's other entry points on the same workload
(or the one named): the fused epilogue (alpha 0.5, beta 1, with C and a
bias), the stream-K form (default workload 1024 x 1024 x 16384), bfloat16
storage, FP8 E4M3 operands quantised from normal values with a per-tensor
scale, and FP8 with per-channel weight scales.

Prints one JSON line with the metric, a roofline object for the GEMM kernel
(achieved TFLOP/s from HIP events on the launch stream, against the MI355X
dense MFMA peak of the path's operand type) and a CPU baseline (the oracle,
on a bounded sample of the same workload, on this host's cores).
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

# MI355X dense MFMA peaks: 256 CUs x FLOP/clock/CU x 2.4 GHz; fp16 and
# bf16 4096 FLOP/clock/CU (AMD's published 2.5 PFLOP/s dense figure), FP8
# twice that (5.0 PFLOP/s).
PEAK_FP16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_FP8_TFLOPS = 2 * PEAK_FP16_TFLOPS
PEAK_HBM_GBS = 8000.0
CSRC = ROOT / "dense_gemm_18_amd" / "csrc"
# Sources of each path's kernels (their hash tells whether recorded counters
# still describe the kernel).
PATH_SOURCES = {
    "f16": ["gemm_kernels.h", "gemm_nt_f16.hip"],
    "f16_ws": ["gemm_kernels.h", "gemm_nt_f16.hip"],
    "f16_ex": ["gemm_kernels.h", "gemm_nt_f16_ex.hip"],
    "f16_acc16": ["gemm_kernels.h", "gemm_nt_f16_acc16.hip"],
    "bf16": ["gemm_kernels.h", "gemm_nt_bf16.hip"],
    "fp8": ["gemm_kernels.h", "gemm_fp8.h", "gemm_nt_fp8.hip"],
    "fp8_cs": ["gemm_kernels.h", "gemm_fp8.h", "gemm_nt_fp8.hip"],
}
KERNEL_SOURCES = [CSRC / f for f in PATH_SOURCES["f16"]]


def tflops(M: int, N: int, K: int, seconds: float) -> float:
    """TFLOPS = 2*M*N*K / (t * 1e12): one multiply-add counts two."""
    return 2.0 * M * N * K / (seconds * 1e12)


def algorithmic_bytes(M: int, N: int, K: int, elem: int = 2, extra: float = 0.0) -> float:
    """A and B read once (elem bytes per element), D written once (2-byte),
    plus `extra` bytes (the fused epilogue's C and bias)."""
    return elem * (M * K + N * K) + 2.0 * M * N + extra


def kernel_source_hash(path: str = "f16") -> str:
    """Hash of a path's kernel sources' code: comments and whitespace are
    dropped, so only a change to the code itself invalidates recorded
    counters."""
    text = "\n".join((CSRC / f).read_text() for f in PATH_SOURCES[path])
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_summary(path: str, workload: str) -> Path:
    return ROOT / "profiles" / f"gemm_nt_{path}_{workload}_traffic.md"


def recorded_traffic(path: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    f = traffic_summary(path, workload)
    if not f.exists():
        return None
    text = f.read_text()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not b or h.group(1) != kernel_source_hash(path):
        return None
    return float(b.group(1))


def _oracle_rows(rows_fn, M, N, K, threads: int, budget_s: float):
    """Whole rows of D through the oracle until all M rows or ~budget_s;
    returns (rows, seconds)."""
    chunk = 64
    rows = 0
    t0 = time.perf_counter()
    while rows < M and time.perf_counter() - t0 < budget_s:
        r1 = min(M, rows + chunk)
        rows_fn(rows, r1, threads)
        rows = r1
    return rows, time.perf_counter() - t0


def cpu_baseline(rows_fn, M, N, K, budget_s: float = 12.0, single_thread: bool = False) -> dict:
    """The oracle (untuned) on whole rows of D until ~budget_s of CPU work;
    rows_fn(r0, r1, threads) computes rows r0 .. r1-1.  single_thread: also
    time it on one thread (the small workloads, whose whole D a single core
    computes within the budget)."""
    import oracle
    threads = oracle.threads_available()
    rows, dt = _oracle_rows(rows_fn, M, N, K, threads, budget_s)
    out = {
        "value": tflops(rows, N, K, dt),
        "unit": "TFLOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{rows} full rows of D ({rows}x{N}x{K}, {rows * N * K:.3e} MACs) in {dt:.1f} s",
        "host": host_cpu(),
    }
    if single_thread:
        rows1, dt1 = _oracle_rows(rows_fn, M, N, K, 1, budget_s)
        out["single_thread"] = {
            "value": tflops(rows1, N, K, dt1),
            "unit": "TFLOPS",
            "cores": 1,
            "sample": f"{rows1} full rows of D ({rows1 * N * K:.3e} MACs) in {dt1:.2f} s",
        }
    return out


def host_cpu() -> dict:
    """The host's CPU model and how many of its cores this process may use."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0))}


class ClockSampler:
    """Shader clock and socket power while the benchmark runs.

    amd-smi runs as a child process in watch mode (one sample of every XCD's
    GFX clock and the socket power per second), started before this process
    touches the GPU and stopped (its process group) once the GPU work is
    done.  A reader thread stamps each line with the time it arrived, so the
    samples that fall inside the loaded part of the run can be picked out.
    The power cap comes from `rocm-smi --showmaxpower` (amd-smi's static
    limit query is not offered on a guest), run first by the same child."""

    CMD = ("rocm-smi -d 0 --showmaxpower --json; echo __METRIC__; "
           "amd-smi metric -g 0 -c -p -w 1")

    def __init__(self):
        import subprocess
        import threading
        self.lines = []
        self.error = None
        self.proc = None
        env = dict(os.environ, PYTHONUNBUFFERED="1")
        try:
            self.proc = subprocess.Popen(["bash", "-c", self.CMD], stdout=subprocess.PIPE,
                                         stderr=subprocess.STDOUT, text=True, env=env,
                                         start_new_session=True)
        except OSError as e:
            self.error = f"amd-smi not started: {e}"
            return
        self.reader = threading.Thread(target=self._read, daemon=True)
        self.reader.start()

    def _read(self):
        for line in self.proc.stdout:
            self.lines.append((time.monotonic(), line.rstrip("\n")))

    def stop(self):
        import signal
        if self.proc is None or self.proc.returncode is not None:
            return
        try:
            os.killpg(self.proc.pid, signal.SIGTERM)
        except OSError:
            pass
        try:
            self.proc.wait(timeout=10)
        except Exception:
            os.killpg(self.proc.pid, signal.SIGKILL)
            self.proc.wait(timeout=10)
        self.reader.join(timeout=5)

    def parse(self):
        """[{"t", "gfx": [MHz per XCD], "power": W}] per watch sample, and
        the power limits (name -> W) from the static query."""
        samples, limits = [], {}
        cur, section, ppt, in_metric = None, "", "", False
        for t, line in self.lines:
            s = line.strip()
            if s == "__METRIC__":
                in_metric = True
                continue
            if not in_metric:
                m = re.search(r'Max Graphics Package Power \(W\)"?\s*:\s*"?([0-9.]+)', s)
                if m:
                    limits["max_graphics_package_power"] = float(m.group(1))
                m = re.match(r"^(PPT\d+):", s)
                if m:
                    ppt = m.group(1)
                m = re.match(r"^(\w*POWER\w*):\s*([0-9.]+)\s*W\b", s)
                if m:
                    limits[f"{ppt}.{m.group(1)}" if ppt else m.group(1)] = float(m.group(2))
                continue
            if re.match(r"^GPU:\s*\d+", s):
                if cur is not None:
                    samples.append(cur)
                cur = {"t": t, "gfx": [], "power": None}
                continue
            if cur is None:
                continue
            m = re.match(r"^(GFX_\d+):\s*(.*)$", s)
            if m:
                section = m.group(1)
                m2 = re.match(r"CLK:\s*([0-9.]+)\s*MHz", m.group(2))
                if m2:
                    cur["gfx"].append(float(m2.group(1)))
                    section = ""
                continue
            if re.match(r"^[A-Z0-9_]+:\s*$", s):
                section = ""
                continue
            m = re.match(r"^CLK:\s*([0-9.]+)\s*MHz", s)
            if m and section.startswith("GFX_"):
                cur["gfx"].append(float(m.group(1)))
                cur["t"] = t
                section = ""
                continue
            m = re.match(r"^SOCKET_POWER:\s*([0-9.]+)\s*W", s)
            if m:
                cur["power"] = float(m.group(1))
        if cur is not None:
            samples.append(cur)
        return [x for x in samples if x["gfx"] or x["power"] is not None], limits

    def report(self, t0: float, t1: float, peak: float, value: float) -> dict:
        """Clock and power over the samples read between t0 and t1 (the
        loaded part of the run), and the value as a fraction of the peak at
        the mean clock held there."""
        rocm = ""
        try:
            rocm = Path("/opt/rocm/.info/version").read_text().strip()
        except OSError:
            pass
        out = {"source": "amd-smi metric -g 0 -c -p -w 1 (and rocm-smi --showmaxpower), a child "
                         "process started before the GPU was first used", "rocm": rocm}
        if self.error:
            out["error"] = self.error
            return out
        samples, limits = self.parse()
        out["power_limits_w"] = limits
        if not limits:
            # the static query's text, when its layout did not parse
            static = []
            for _, ln in self.lines:
                if ln.strip() == "__METRIC__":
                    break
                if ln.strip():
                    static.append(ln.strip())
            out["power_limit_text"] = static[:16]
        inside = [x for x in samples if t0 <= x["t"] <= t1 and x["gfx"]]
        out["samples_total"] = len(samples)
        out["samples_under_load"] = len(inside)
        if not inside:
            out["error"] = "no amd-smi sample fell inside the loaded part of the run"
            out["raw_tail"] = [ln for _, ln in self.lines[-6:]]
            return out
        clks = [c for x in inside for c in x["gfx"]]
        pw = [x["power"] for x in inside if x["power"] is not None]
        mean = sum(clks) / len(clks)
        out.update({
            "gfx_mhz_mean": round(mean, 1), "gfx_mhz_min": min(clks), "gfx_mhz_max": max(clks),
            "gfx_mhz_per_xcd_last": inside[-1]["gfx"],
            "socket_power_w_mean": round(sum(pw) / len(pw), 1) if pw else None,
            "socket_power_w_max": max(pw) if pw else None,
            "spec_mhz": 2400,
            "peak_at_held_clock": round(peak * mean / 2400.0, 1),
            "frac_of_peak_at_held_clock": round(value / (peak * mean / 2400.0), 4),
        })
        return out


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


def setup_path(path, w, torch, dev, binding, wl) -> dict:
    """Inputs resident on the GPU and one step of the chosen entry point,
    with what the report needs about it."""
    import numpy as np

    M, N, K = w.M, w.N, w.K
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    dD = torch.empty((M, N), dtype=torch.float16, device=dev)
    pd = dD.data_ptr()
    fp16_inputs = {"A": f"{w.a_dist} fp16, seed {w.seeds[0]}",
                   "B": f"{w.b_dist} fp16, seed {w.seeds[1]}"}

    def check(rc, what):
        if rc != binding.GEMM_OK:
            raise RuntimeError(f"{what}: {binding.gemm_nt_f16_strerror(rc)}")

    keep = [dD]              # device buffers the steps use stay alive with P
    P = {"keep": keep, "peak": PEAK_FP16_TFLOPS, "bytes": algorithmic_bytes(M, N, K),
         "dtype": "fp16", "inputs": fp16_inputs, "tile": list(binding.gemm_nt_f16_tile(M, N, K)[:3])}
    if path in ("f16", "f16_ws", "f16_ex", "f16_acc16"):
        A, B = wl.random_inputs(w)
        dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        pa, pb = dA.data_ptr(), dB.data_ptr()
        P["tensors"] = (dA, dB)
        keep += [dA, dB]
    if path == "f16":
        import oracle
        # HBM-bound shapes (below the ridge point) whose operands are large
        # (32 MB or more) rotate over independent copies of A and B totalling
        # more than 512 MB, so that the 256 MB MALL cannot serve the next
        # launch's operands: every launch streams them from HBM.  Compute-
        # bound shapes, and problems small enough to be latency-bound, are
        # timed warm.
        sets = [(pa, pb)]
        per_set = 2 * (M * K + N * K)
        if (2.0 * M * N * K / P["bytes"] < PEAK_FP16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
                and per_set >= (32 << 20)):
            for _ in range(max(2, -(-(512 << 20) // per_set) + 1) - 1):
                cA, cB = dA.clone(), dB.clone()
                keep += [cA, cB]
                sets.append((cA.data_ptr(), cB.data_ptr()))
            P["inputs"] = dict(fp16_inputs, operand_copies=len(sets),
                               operand_bytes_rotated=len(sets) * per_set)
        turn = [0]

        def step_f16():
            a, b = sets[turn[0] % len(sets)]
            turn[0] += 1
            check(binding.gemm_nt_f16(a, b, pd, M, N, K, sptr), "gemm_nt_f16")

        P.update(entry="gemm_nt_f16",
                 metric=("fp16 GEMM TFLOPS (2MNK/t) at 8192^3; % of MI355X dense fp16 MFMA peak"
                         if w.name == wl.HEADLINE else
                         f"fp16 GEMM TFLOPS (2MNK/t), {M}x{N}x{K}"),
                 step=step_f16,
                 cpu_rows=lambda r0, r1, t: oracle.gemm_nt_f16(A[r0:r1], B, threads=t))
    elif path == "f16_ws":
        import oracle
        need = max(binding.gemm_nt_f16_ws_size(M, N, K), 256)
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        keep.append(ws)
        bm, bn, wg, skt = binding.gemm_nt_f16_ws_tile(M, N, K)
        P.update(entry="gemm_nt_f16_ws", tile=[bm, bn, 64], stream_k_tiles=skt,
                 metric=f"fp16 GEMM TFLOPS (2MNK/t), stream-K form, {M}x{N}x{K}",
                 step=lambda: check(binding.gemm_nt_f16_ws(pa, pb, pd, M, N, K, ws.data_ptr(),
                                                           need, sptr), "gemm_nt_f16_ws"),
                 cpu_rows=lambda r0, r1, t: oracle.gemm_nt_f16(A[r0:r1], B, threads=t))
        P["inputs"] = dict(fp16_inputs, workspace_bytes=need, stream_k_tiles=skt,
                           workgroups=wg)
    elif path == "f16_acc16":
        import oracle
        bm, bn, lb = binding.gemm_nt_f16_acc16_kernel(pa, pb, M, N, K)
        P.update(entry="gemm_nt_f16_acc16", tile=[bm, bn, 64], accumulate="fp16 (64-wide chunks)",
                 metric=f"fp16 GEMM TFLOPS (2MNK/t) with an fp16 running sum, {M}x{N}x{K}",
                 step=lambda: check(binding.gemm_nt_f16_acc16(pa, pb, pd, M, N, K, sptr),
                                    "gemm_nt_f16_acc16"),
                 cpu_rows=lambda r0, r1, t: oracle.gemm_nt_f16_acc16(A[r0:r1], B, threads=t))
    elif path == "f16_ex":
        import oracle
        rng = np.random.default_rng(w.seeds[0] + 77)
        C = rng.uniform(-1.0, 1.0, size=(M, N)).astype(np.float16)
        bias = rng.uniform(-1.0, 1.0, size=N).astype(np.float16)
        dC, dbias = torch.from_numpy(C).to(dev), torch.from_numpy(bias).to(dev)
        keep += [dC, dbias]
        alpha, beta = 0.5, 1.0
        P.update(entry="gemm_nt_f16_ex", bytes=algorithmic_bytes(M, N, K, extra=2.0 * (M * N + N)),
                 metric=f"fp16 GEMM TFLOPS (2MNK/t) with fused alpha/beta/bias epilogue, "
                        f"{M}x{N}x{K}",
                 step=lambda: check(binding.gemm_nt_f16_ex(pa, pb, dC.data_ptr(), dbias.data_ptr(),
                                                           pd, M, N, K, alpha, beta, sptr),
                                    "gemm_nt_f16_ex"),
                 cpu_rows=lambda r0, r1, t: oracle.gemm_nt_f16_ex(A[r0:r1], B, C[r0:r1], bias,
                                                                  alpha, beta))
        P["inputs"] = dict(fp16_inputs, C="uniform[-1,1] fp16", bias="uniform[-1,1] fp16",
                           alpha=alpha, beta=beta)
    elif path == "bf16":
        import oracle
        A, B = wl.bf16_uniform(w.seeds[0], M, N, K)
        dA = torch.from_numpy(A.view(np.int16)).to(dev)
        dB = torch.from_numpy(B.view(np.int16)).to(dev)
        pa, pb = dA.data_ptr(), dB.data_ptr()
        keep += [dA, dB]
        P.update(entry="gemm_nt_bf16", dtype="bf16",
                 metric=f"bf16 GEMM TFLOPS (2MNK/t), {M}x{N}x{K}; % of MI355X dense bf16 MFMA peak",
                 step=lambda: check(binding.gemm_nt_bf16(pa, pb, pd, M, N, K, sptr), "gemm_nt_bf16"),
                 cpu_rows=lambda r0, r1, t: oracle.gemm_nt_bf16(A[r0:r1], B, threads=t))
        P["inputs"] = {"A": f"uniform[-1,1] bf16, seed {w.seeds[0]}",
                       "B": f"uniform[-1,1] bf16, seed {w.seeds[0]} (second draw)"}
    elif path == "fp8":
        import oracle
        A, B, scale = wl.fp8_normal(w.seeds[0], M, N, K)
        dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        pa, pb = dA.data_ptr(), dB.data_ptr()
        keep += [dA, dB]
        e4 = binding.GEMM_FP8_E4M3
        P.update(entry="gemm_nt_fp8", dtype="fp8_e4m3", peak=PEAK_FP8_TFLOPS,
                 bytes=algorithmic_bytes(M, N, K, elem=1),
                 tile=list(binding.gemm_nt_fp8_tile(M, N, K, True)) + [128],
                 metric=f"FP8 E4M3 GEMM TFLOPS (2MNK/t), {M}x{N}x{K}, fp16 out; % of MI355X "
                        "dense FP8 MFMA peak",
                 step=lambda: check(binding.gemm_nt_fp8(pa, pb, pd, M, N, K, scale, e4, e4, sptr),
                                    "gemm_nt_fp8"),
                 cpu_rows=lambda r0, r1, t: oracle.gemm_nt_fp8(A[r0:r1], B, scale, threads=t))
        P["inputs"] = {"A": f"standard normal quantised to E4M3 (per-tensor scale), seed "
                            f"{w.seeds[0]}",
                       "B": "standard normal quantised to E4M3 (per-tensor scale), same stream",
                       "scale": scale}
    elif path == "fp8_cs":
        import oracle
        A, B, sa, sb = wl.fp8_channelwise(w.seeds[0], M, N, K)
        dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        dS = torch.from_numpy(sb).to(dev)
        pa, pb, ps = dA.data_ptr(), dB.data_ptr(), dS.data_ptr()
        keep += [dA, dB, dS]
        e4 = binding.GEMM_FP8_E4M3
        P.update(entry="gemm_nt_fp8_cs", dtype="fp8_e4m3", peak=PEAK_FP8_TFLOPS,
                 bytes=algorithmic_bytes(M, N, K, elem=1, extra=4.0 * N),
                 tile=list(binding.gemm_nt_fp8_tile(M, N, K, True)) + [128],
                 metric=f"FP8 E4M3 GEMM TFLOPS (2MNK/t) with per-channel weight scales, "
                        f"{M}x{N}x{K}, fp16 out; % of MI355X dense FP8 MFMA peak",
                 step=lambda: check(binding.gemm_nt_fp8_cs(pa, pb, pd, M, N, K, sa, ps, e4, e4,
                                                           sptr), "gemm_nt_fp8_cs"),
                 cpu_rows=lambda r0, r1, t: oracle.gemm_nt_fp8_cs(A[r0:r1], B, sa, sb, threads=t))
        P["inputs"] = {"A": f"standard normal quantised to E4M3 (per-tensor scale), seed "
                            f"{w.seeds[0]}",
                       "B": "N(0, 0.02^2) weights, rows scaled by U[0.25, 4], quantised to E4M3 "
                            "with one scale per row, same stream",
                       "a_scale": sa}
    else:
        raise ValueError(path)
    return P


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    # ~0.1 s of warm-up brings the clock to its steady level under the power
    # limit (the first tens of milliseconds of load run slower); the timed
    # region then spans well over 0.2 s.
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None, help="workload name (default: the 8192^3 GEMM)")
    ap.add_argument("--path", default="f16", choices=sorted(PATH_SOURCES),
                    help="entry point to time (default: gemm_nt_f16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prewarm", type=float, default=3.0,
                    help="seconds of back-to-back launches before the warm-up steps, so that "
                         "the clock reaches the level it holds under this load (the first "
                         "~0.1 s run slower); not part of the timed region")
    ap.add_argument("--clock", action=argparse.BooleanOptionalAction, default=True,
                    help="sample the shader clock and socket power with amd-smi (a child "
                         "process started before the GPU is touched); off under profilers")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    ap.add_argument("--sustain", type=float, default=0.0,
                    help="only run the GEMM back to back for this many seconds (for sampling "
                         "clock and power with amd-smi); prints the achieved TFLOPS")
    ap.add_argument("--torch-context", action=argparse.BooleanOptionalAction, default=True,
                    help="also time torch.nn.functional.linear (hipBLASLt) on the same inputs "
                         "(fp16 path only; context, never a reference)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this GEMM path is "
              "single-GPU and has no multi-GPU mode.", file=sys.stderr)
        return 2

    # The sampler starts before torch touches the GPU, and is always stopped.
    sampler = ClockSampler() if args.clock and not args.copy_calibration else None
    try:
        return run(args, sampler)
    finally:
        if sampler is not None:
            sampler.stop()


def run(args, sampler) -> int:
    import torch

    if args.copy_calibration:
        return copy_calibration(torch)

    from dense_gemm_18_amd import binding
    from dense_gemm_18_amd import build as hip_build
    from dense_gemm_18_amd import workloads as wl

    if not binding.library_path().exists():
        hip_build.build()
    path = args.path
    name = args.workload or ("deep_1024x1024x16384" if path == "f16_ws" else wl.HEADLINE)
    w = wl.WORKLOADS[name]
    M, N, K = w.M, w.N, w.K
    dev = torch.device("cuda:0")
    P = setup_path(path, w, torch, dev, binding, wl)
    step = P["step"]
    stream = torch.cuda.current_stream(dev)        # the stream every launch goes to

    t_load = time.monotonic()
    prewarm_calls = 0
    if args.prewarm > 0 and args.sustain <= 0:
        while time.monotonic() - t_load < args.prewarm:
            for _ in range(20):
                step()
            torch.cuda.synchronize(dev)
            prewarm_calls += 20
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

    # Timed region: exactly `steps` calls, synchronised on both sides, with
    # one HIP event pair on the launch stream around all of them: the GPU
    # time per launch (back-to-back launches, as rocprofv3's kernel trace
    # sees them) gives roofline.achieved.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    avg_kernel_s = ev0.elapsed_time(ev1) / args.steps / 1e3
    ms_per_step = wall / args.steps * 1e3

    # Spread of single launches (after the timed region, not part of it):
    # each launch bracketed by its own events, which adds their overhead.
    n_single = min(args.steps, 100)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_single)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_single)]
    for i in range(n_single):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize(dev)
    kernel_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    median_ms = kernel_ms[len(kernel_ms) // 2]
    t_unload = time.monotonic()

    value = tflops(M, N, K, wall / args.steps)
    achieved = tflops(M, N, K, avg_kernel_s)
    peak = P["peak"]
    traffic = recorded_traffic(path, name)
    # The kernel's bound: MFMA when its arithmetic intensity (algorithmic
    # FLOP per algorithmic byte) is above the ridge point peak / HBM
    # bandwidth, else HBM (the skinny linear-layer shapes).
    intensity = 2.0 * M * N * K / P["bytes"]
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity >= ridge:
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    else:
        gbs = P["bytes"] / avg_kernel_s / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "tflops": round(achieved, 2),
                "pct_of_mfma_peak": round(100.0 * achieved / peak, 2)}
    roof["arithmetic_intensity_flop_per_byte"] = round(intensity, 1)
    roof["ridge_flop_per_byte"] = round(ridge, 1)
    props = torch.cuda.get_device_properties(dev)
    out = {
        "metric": P["metric"],
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": P["dtype"],
        "data": "synthetic",
        "config": {
            "workload": name, "M": M, "N": N, "K": K, "entry_point": P["entry"],
            **P["inputs"],
            "accumulate": P.get("accumulate", "fp32"),
            "layout": "A MxK, B NxK (D = A B^T), row-major",
            "tile": P["tile"],
        },
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {
            **roof,
            "traffic": traffic,
            "kernel_ms_avg": round(avg_kernel_s * 1e3, 5),
            "single_launch_ms_median": round(median_ms, 5),
            "single_launch_ms_min": round(kernel_ms[0], 5),
            "single_launch_ms_max": round(kernel_ms[-1], 5),
            "algorithmic_flops_per_launch": 2.0 * M * N * K,
            "algorithmic_bytes_per_launch": P["bytes"],
            "hbm_gbs_at_algorithmic_bytes": round(P["bytes"] / avg_kernel_s / 1e9, 1),
        },
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
        "kernel_source_sha256_16": kernel_source_hash(path),
        "prewarm": {"seconds": args.prewarm, "launches": prewarm_calls},
    }
    if args.torch_context and path == "f16":
        dA, dB = P["tensors"]
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
    if name == wl.HEADLINE and path in ("f16", "f16_acc16"):
        # the pages' own figures for this workload, on other hardware:
        # context, not a reference (page 1, "如何用 Croqtile 一步步优化矩阵乘法
        # 内核", sections "性能一览" and "SOTA 对比"; its tuned kernel
        # accumulates in fp16)
        out["context_published"] = {
            "hardware": "NVIDIA H800 PCIe", "cublas_torch_mm_tflops": 447.5,
            "tuned_kernel_fp16_accumulate_tflops": 489.9}
    if sampler is not None:
        sampler.stop()
        # samples from 1 s into the load (the clock settles) to the end of the
        # GPU work; amd-smi reports each sample averaged over its interval
        out["clock"] = sampler.report(t_load + 1.0, t_unload + 1.0, peak, value)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(P["cpu_rows"], M, N, K,
                                           single_thread=M * N * K <= 1024 ** 3)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
