"""GPU parity of the stream-K entry point gemm_nt_f16_ws against the oracle.

Shapes are chosen so that the persistent kernel runs with 3 to 32
contributors per tile, pieces that cross tile boundaries, a single tile
row, rows not 16-byte aligned with a K tail, and the skinny shapes' 64 x 32,
32 x 64 and 64 x 64 tiles.  The
bar is the one of the plain entry point: integer inputs bit-exact, random
inputs within 2^-10 |D_ref| + 1e-3 sqrt(K).  The summation order is fixed
per shape, so repeated calls must agree bit for bit, and the workspace must
come back with its flag words zero.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from dense_gemm_18_amd import binding
from dense_gemm_18_amd import workloads as wl
from tests.gpu_util import assert_bitexact, assert_tolerance, device, note, run_gemm_ws

pytestmark = pytest.mark.gpu

SHAPES = [
    (1024, 1024, 12288),     # 64 tiles, 3 contributors each
    (768, 768, 12288),       # 36 tiles, pieces cross tile boundaries
    (512, 640, 16384),       # 20 tiles, up to 12 contributors each
    (900, 1000, 12290),      # ragged M, N; rows 4-byte aligned, a K tail
    (512, 640, 12351),       # odd K: rows 2-byte aligned, first-step fix-up
    (768, 1024, 12296),      # 16-byte loads and a K tail (only step 0 masked)
    (100, 8192, 32768),      # one tile row, K = 32768
    # skinny shapes (M or N <= 64)
    (64, 2048, 8192),        # 64 x 32 tiles, 4 contributors each
    (2048, 64, 8192),        # 32 x 64 tiles
    (64, 4096, 4096),        # 64 x 64 tiles
    (8192, 64, 8192),        # 64 x 64 tiles where the plain grid fills the CUs
    (64, 2000, 8200),        # ragged N, a K tail
    (1, 4096, 4096),         # one row
    (48, 3000, 4096),        # ragged M and N
    (64, 256, 16384),        # 32 contributors per tile
]


@pytest.fixture(scope="module", autouse=True)
def _library_present():
    assert binding.library_path().exists(), "libgemm18.so not built"


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_stream_k_integer_bitexact(M, N, K):
    assert binding.gemm_nt_f16_ws_tile(M, N, K)[3] > 0, "shape must take the stream-K plan"
    A, B = wl.integer_free(6000 + K, M, N, K)
    note(f"stream-K integer {M}x{N}x{K} plan {binding.gemm_nt_f16_ws_tile(M, N, K)}")
    d = run_gemm_ws(A, B)
    ref = oracle.gemm_nt_f16(A, B)
    assert np.abs(oracle.decode(ref)).max() <= 2048
    assert_bitexact(d, ref, f"stream-K {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_stream_k_random_tolerance(M, N, K):
    A, B = wl.uniform_inputs(7000 + K, M, N, K)
    note(f"stream-K random {M}x{N}x{K}")
    d = run_gemm_ws(A, B)
    assert_tolerance(d, oracle.gemm_nt_f16(A, B), K, f"stream-K random {M}x{N}x{K}")


def test_stream_k_deterministic_and_reusable():
    import torch
    dev = device()
    ws = torch.zeros(max(binding.gemm_nt_f16_ws_size(*s) for s in SHAPES[:3]), dtype=torch.uint8,
                     device=dev)
    A1, B1 = wl.uniform_inputs(8001, 768, 768, 12288)
    A2, B2 = wl.uniform_inputs(8002, 1024, 1024, 12288)
    note("stream-K reuse: shape 1 twice, shape 2, shape 1")
    d1 = run_gemm_ws(A1, B1, ws, repeat=2)
    d2 = run_gemm_ws(A2, B2, ws)
    d1b = run_gemm_ws(A1, B1, ws)
    assert np.array_equal(d1, d1b)
    assert_tolerance(d2, oracle.gemm_nt_f16(A2, B2), 12288, "stream-K reuse shape 2")
    # header: word 0 counts the calls, word 1 (the done counter) is back to
    # zero, word 2 (timeouts) is clear; flags hold call numbers, never more
    # than the last one
    hdr = ws[:256].cpu().numpy().view(np.uint32)
    assert hdr[0] == 4 and hdr[1] == 0 and hdr[2] == 0, hdr[:4]
    flags = ws[256:256 + 1024].cpu().numpy().view(np.uint32)
    assert flags.max() <= 4 and flags.any()


def test_stream_k_too_small_workspace_runs_plain():
    A, B = wl.integer_free(8100, 1024, 1024, 12288)
    import torch
    ws = torch.zeros(4096, dtype=torch.uint8, device=device())
    note("stream-K with a too-small workspace")
    d = run_gemm_ws(A, B, ws)
    assert_bitexact(d, oracle.gemm_nt_f16(A, B), "too-small workspace")


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 65536), (2048, 2048, 4096)])
def test_stream_k_sampled_large(M, N, K):
    # K = 65536 (1024 K-steps split over 4 workgroups per tile) and a
    # plain-path shape through the same entry point; sampled entries plus
    # the rows at tile edges against the oracle.
    A, B = wl.uniform_inputs(8200 + K, M, N, K)
    note(f"stream-K sampled {M}x{N}x{K}")
    d = run_gemm_ws(A, B, repeat=2)
    rng = np.random.default_rng(8300)
    flat = rng.choice(M * N, 4096, replace=False)
    rows, cols = flat // N, flat % N
    er = wl.edge_lines(M, 128)
    rr = np.repeat(er, N)
    rc = np.tile(np.arange(N), er.size)
    rows = np.concatenate([rows, rr])
    cols = np.concatenate([cols, rc])
    ref = oracle.gemm_nt_f16_entries(A, B, rows, cols)
    assert_tolerance(d[rows, cols], ref, K, f"stream-K sampled {M}x{N}x{K}")
