"""Overlapping calls: the entry points keep no per-call state in the library,
so calls on different streams, and calls from different host threads, may
run at the same time.  Every call here writes its own output; after all of
them have finished, each output must equal, bit for bit, the same call made
alone, and that in turn equals the oracle (integer inputs, so the fp32 sums
are exact and both sides round the same value once).

The cases cover the 256 x 256, 256 x 128, 128 x 128 and 64 x 64 direct-to-LDS tiles,
rows that are not 16-byte aligned on the direct loads and on the register-
staged ones, the fp16-accumulating and FP8 entry points, and
the stream-K form (128 x 128 and skinny 64 x 32 plans).  The stream-K
calls overlap the others but never each other: each grid expects to get
every CU once the kernels around it finish, so all of them go on one
stream, as the header asks.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest

import oracle
from dense_gemm_18_amd import binding
from dense_gemm_18_amd import workloads as wl
from tests.gpu_util import note

pytestmark = pytest.mark.gpu

ROUNDS = 4


class Case:
    """One call with its device inputs, an output per round and the oracle's
    result."""

    def __init__(self, name, M, N, K, seed, kind="f16"):
        import torch
        dev = torch.device("cuda:0")
        self.name, self.M, self.N, self.K, self.kind = name, M, N, K, kind
        if kind == "fp8":
            A, B = wl.fp8_integers(seed, M, N, K, 0, 1)
            self.ref = oracle.gemm_nt_fp8(A, B, 0.25, a_e5m2=False, b_e5m2=True)
        elif kind == "acc16":
            rng = np.random.default_rng(seed)
            A = rng.integers(4, 9, size=(M, K)).astype(np.float16)
            B = rng.integers(4, 9, size=(N, K)).astype(np.float16)
            self.ref = oracle.gemm_nt_f16_acc16(A, B)
        else:
            A, B = wl.integer_free(seed, M, N, K, -2, 2)
            self.ref = oracle.gemm_nt_f16(A, B)
        if kind == "reg":
            # odd K on a skinny shape: the register-staged kernel
            assert K % 2 == 1 and min(M, N) <= 64
        self.dA = torch.from_numpy(np.ascontiguousarray(A).view(np.uint8)).to(dev)
        self.dB = torch.from_numpy(np.ascontiguousarray(B).view(np.uint8)).to(dev)
        self.outs = [torch.empty((M, N), dtype=torch.int16, device=dev) for _ in range(ROUNDS)]
        self.ws = None
        if kind == "ws":
            need = binding.gemm_nt_f16_ws_size(M, N, K)
            assert need > 0, "the stream-K case must plan stream-K"
            self.ws_bytes = need
            self.ws = torch.zeros(need, dtype=torch.uint8, device=dev)

    def reset(self):
        # a NaN pattern no call writes, so an output a call skipped shows
        for out in self.outs:
            out.fill_(0x7E5A)

    def call(self, r, stream):
        a, b, d = self.dA.data_ptr(), self.dB.data_ptr(), self.outs[r].data_ptr()
        M, N, K = self.M, self.N, self.K
        if self.kind == "fp8":
            return binding.gemm_nt_fp8(a, b, d, M, N, K, 0.25, binding.GEMM_FP8_E4M3,
                                       binding.GEMM_FP8_E5M2, stream)
        if self.kind == "acc16":
            return binding.gemm_nt_f16_acc16(a, b, d, M, N, K, stream)
        if self.kind == "ws":
            return binding.gemm_nt_f16_ws(a, b, d, M, N, K, self.ws.data_ptr(), self.ws_bytes,
                                          stream)
        return binding.gemm_nt_f16(a, b, d, M, N, K, stream)

    def check(self):
        for r, out in enumerate(self.outs):
            got = out.cpu().numpy().view(np.uint16)
            bad = np.count_nonzero(got != self.ref)
            assert bad == 0, f"{self.name} round {r}: {bad} entries differ from the oracle"


@pytest.fixture(scope="module")
def cases():
    return [Case("256x256 tile", 2900, 4100, 512, 24001),
            Case("128x128 tile", 1000, 1100, 576, 24002),
            Case("64x64 tile", 64, 3000, 448, 24003),
            Case("unaligned rows", 700, 900, 201, 24004),
            Case("register-staged", 64, 3000, 201, 24008, "reg"),
            Case("fp16 accumulation", 1000, 1100, 320, 24005, "acc16"),
            Case("fp8", 1000, 1100, 1024, 24006, "fp8"),
            Case("stream-K", 512, 640, 12352, 24007, "ws"),
            Case("256x128 tile", 2100, 2200, 1032, 24009),
            Case("skinny stream-K", 64, 2048, 8192, 24010, "ws")]


def test_calls_on_overlapping_streams(cases):
    import torch
    for c in cases:
        c.reset()
    torch.cuda.synchronize()
    for c in cases:
        note(f"concurrency: {c.name} {c.M}x{c.N}x{c.K} alone")
        assert c.call(0, torch.cuda.current_stream().cuda_stream) == binding.GEMM_OK
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    note("concurrency: every case on three streams, no waits between calls")
    for r in range(1, ROUNDS):
        for i, c in enumerate(cases):
            s = streams[0] if c.kind == "ws" else streams[(i + r) % len(streams)]
            assert c.call(r, s.cuda_stream) == binding.GEMM_OK
    torch.cuda.synchronize()
    for c in cases:
        c.check()


def test_calls_from_threads(cases):
    # one host thread per case, except that the stream-K cases share one
    # thread (and its stream), as they share the GPU's CUs
    import torch
    for c in cases:
        c.reset()
    torch.cuda.synchronize()
    groups = [[c] for c in cases if c.kind != "ws"] + [[c for c in cases if c.kind == "ws"]]
    errors = []
    start = threading.Barrier(len(groups))

    def worker(group):
        try:
            s = torch.cuda.Stream()
            start.wait()
            for r in range(ROUNDS):
                for c in group:
                    rc = c.call(r, s.cuda_stream)
                    if rc != binding.GEMM_OK:
                        errors.append(f"{c.name}: rc {rc}")
            s.synchronize()
        except Exception as e:           # reported below, on the main thread
            errors.append(f"{group[0].name}: {e!r}")

    note(f"concurrency: {len(groups)} host threads, {ROUNDS} rounds each")
    threads = [threading.Thread(target=worker, args=(g,)) for g in groups]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for c in cases:
        c.check()
