"""GPU parity of the bfloat16 product gemm_nt_bf16 against the oracle.

Integer inputs are bit-exact at any K: the fp32 sum of small integers is
exact on the GPU, the fp64 sum is exact in the oracle, and both round the
same exact value once to bfloat16.  Random inputs must satisfy
|D - D_ref| <= 2^-7 |D_ref| + 1e-3 sqrt(K) (one bfloat16 rounding step, which
is 2^-8 relative at most, on either side, plus fp32 accumulation drift).
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from dense_gemm_18_amd import binding
from dense_gemm_18_amd import workloads as wl
from tests.gpu_util import note, run_gemm_bf16

pytestmark = pytest.mark.gpu

# 256x256 (both B rings), 128x128, 64x64, rows not 16-byte aligned (K = 130, 37)
SHAPES = [(2900, 4100, 136), (2900, 4100, 512), (2100, 2200, 1032), (1100, 1100, 96), (64, 300, 128), (300, 200, 130), (150, 97, 37),
          (1024, 1024, 1024), (64, 3000, 136), (3000, 40, 200), (2100, 2200, 200)]


def _check_tol(got, ref, K, what):
    g = oracle.bf16_decode(got)
    r = oracle.bf16_decode(ref)
    bound = 2.0 ** -7 * np.abs(r) + 1e-3 * math.sqrt(K)
    bad = np.flatnonzero(~(np.abs(g - r) <= bound))
    note(f"{what}: bitwise equal {np.mean(got == ref):.4f}, bad {bad.size}")
    assert bad.size == 0, f"{what}: {bad.size} entries outside tolerance, first {bad[:5]}"


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_integer_bitexact(M, N, K):
    A, B = wl.bf16_integers(9700 + K, M, N, K)
    note(f"bf16 integer {M}x{N}x{K}")
    d = run_gemm_bf16(A, B)
    ref = oracle.gemm_nt_bf16(A, B)
    diff = np.flatnonzero(d != ref)
    assert diff.size == 0, f"{diff.size} entries differ, first {diff[:5]}"


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 64), (1000, 1032, 192), (64, 4096, 512)])
def test_bf16_staged_and_direct_epilogue(M, N, K):
    # whole tiles with D 16-byte aligned and N % 8 == 0 go through LDS; with D
    # only 8-byte aligned (d_off = 4) the same tiles take the direct stores
    A, B = wl.bf16_integers(9900 + M + K, M, N, K)
    ref = oracle.gemm_nt_bf16(A, B)
    note(f"bf16 staged epilogue {M}x{N}x{K}")
    for d_off in (0, 4):
        d = run_gemm_bf16(A, B, d_off=d_off)
        diff = np.flatnonzero(d != ref)
        assert diff.size == 0, f"d_off {d_off}: {diff.size} entries differ, first {diff[:5]}"


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_random_tolerance(M, N, K):
    A, B = wl.bf16_uniform(9800 + K, M, N, K)
    note(f"bf16 random {M}x{N}x{K}")
    _check_tol(run_gemm_bf16(A, B), oracle.gemm_nt_bf16(A, B), K, f"bf16 {M}x{N}x{K}")


def test_bf16_headline_sampled():
    M = N = K = 8192
    A, B = wl.bf16_uniform(9900, M, N, K)
    note("bf16 8192^3 sampled")
    d = run_gemm_bf16(A, B)
    rng = np.random.default_rng(9901)
    flat = rng.choice(M * N, 4096, replace=False)
    rows, cols = flat // N, flat % N
    er = wl.edge_lines(M, 256)
    rows = np.concatenate([rows, np.repeat(er, N)])
    cols = np.concatenate([cols, np.tile(np.arange(N), er.size)])
    ref = oracle.gemm_nt_bf16_entries(A, B, rows, cols)
    _check_tol(d[rows, cols], ref, K, "bf16 8192^3 sampled")


def test_bf16_k_zero():
    A = np.zeros((70, 0), np.uint16)
    B = np.zeros((90, 0), np.uint16)
    note("bf16 K=0")
    assert np.all(run_gemm_bf16(A, B) == 0)
