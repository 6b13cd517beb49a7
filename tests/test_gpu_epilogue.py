"""GPU parity of the fused epilogue gemm_nt_f16_ex against the oracle.

D = alpha * A B^T + beta * C + bias (bias per column), rounded once.  Integer
inputs with dyadic alpha and beta are exact in fp32 on the GPU and in fp64 in
the oracle, so they must match bit for bit on every tile configuration and
load path; random inputs must satisfy |D - D_ref| <= 2^-10 |D_ref| +
1e-3 sqrt(K) |alpha| (the accumulation drift is scaled by alpha; the fp32
epilogue adds rounding far below that).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from dense_gemm_18_amd import binding
from dense_gemm_18_amd import workloads as wl
from tests.gpu_util import assert_bitexact, assert_tolerance, note, run_gemm, run_gemm_ex

pytestmark = pytest.mark.gpu

# (M, N, K, tile the plain path picks): 256x256 16-byte loads, 128x128,
# 64x64 (thin), rows not 16-byte aligned (K = 130, 37, 98)
SHAPES = [(2900, 4100, 136), (2900, 4100, 512), (2100, 2200, 1032), (1100, 1100, 96), (64, 300, 128), (300, 200, 130), (150, 97, 37),
          (3000, 4999, 98), (64, 3000, 136), (3000, 40, 200), (2100, 2200, 200)]
SCALARS = [(2.0, -1.0), (-0.5, 3.0), (1.0, 0.25)]


def _operands(seed, M, N, K):
    A, B = wl.integer_free(seed, M, N, K)
    rng = np.random.default_rng(seed + 1)
    C = rng.integers(-40, 41, size=(M, N)).astype(np.float16)
    bias = rng.integers(-20, 21, size=N).astype(np.float16)
    return A, B, C, bias


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("alpha,beta", SCALARS)
def test_epilogue_integer_bitexact(M, N, K, alpha, beta):
    A, B, C, bias = _operands(9000 + K, M, N, K)
    note(f"epilogue integer {M}x{N}x{K} alpha={alpha} beta={beta}")
    d = run_gemm_ex(A, B, C, bias, alpha, beta)
    ref = oracle.gemm_nt_f16_ex(A, B, C, bias, alpha, beta)
    assert np.abs(oracle.decode(ref)).max() < 2048
    assert_bitexact(d, ref, f"epilogue {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 1024), (1000, 1030, 4100), (333, 222, 1001)])
def test_epilogue_random_tolerance(M, N, K):
    A, B = wl.uniform_inputs(9100 + K, M, N, K)
    rng = np.random.default_rng(9101)
    C = rng.normal(size=(M, N)).astype(np.float16)
    bias = rng.normal(size=N).astype(np.float16)
    alpha, beta = 0.7, -1.3
    note(f"epilogue random {M}x{N}x{K}")
    d = run_gemm_ex(A, B, C, bias, alpha, beta)
    ref = oracle.gemm_nt_f16_ex(A, B, C, bias, alpha, beta)
    assert_tolerance(d, ref, K, f"epilogue random {M}x{N}x{K}", scale=alpha)


def test_epilogue_in_place_c_is_d():
    A, B, C, bias = _operands(9200, 777, 555, 200)
    note("epilogue in place")
    d = run_gemm_ex(A, B, C, bias, 2.0, -1.0, in_place=True)
    assert_bitexact(d, oracle.gemm_nt_f16_ex(A, B, C, bias, 2.0, -1.0), "in place")


def test_epilogue_beta_zero_does_not_read_c():
    A, B, _, bias = _operands(9300, 500, 400, 64)
    C = np.full((500, 400), np.nan, np.float16)
    note("epilogue beta 0 with NaN C")
    d = run_gemm_ex(A, B, C, bias, -2.0, 0.0)
    assert_bitexact(d, oracle.gemm_nt_f16_ex(A, B, None, bias, -2.0, 0.0), "beta 0")


def test_epilogue_k_zero():
    A = np.zeros((70, 0), np.float16)
    B = np.zeros((90, 0), np.float16)
    rng = np.random.default_rng(9400)
    C = rng.normal(size=(70, 90)).astype(np.float16)
    bias = rng.normal(size=90).astype(np.float16)
    note("epilogue K = 0")
    for alpha, beta, cc, bb in [(1.5, 0.5, C, bias), (-1.0, 0.0, None, None), (1.0, 2.0, C, None)]:
        d = run_gemm_ex(A, B, cc, bb, alpha, beta)
        assert_bitexact(d, oracle.gemm_nt_f16_ex(A, B, cc, bb, alpha, beta), f"K=0 {alpha} {beta}")


def test_epilogue_identity_is_plain():
    A, B = wl.uniform_inputs(9500, 1024, 1024, 1024)
    note("epilogue alpha 1 beta 0 no bias")
    assert np.array_equal(run_gemm_ex(A, B), run_gemm(A, B))


def test_epilogue_headline_sampled():
    # 8192^3 on the benchmark's tile: a 64 x 64 block of sampled rows and
    # columns against the oracle's fused epilogue on the same rows of A and B
    w = wl.WORKLOADS[wl.HEADLINE]
    A, B = wl.random_inputs(w)
    rng = np.random.default_rng(9600)
    C = rng.normal(size=(w.M, w.N)).astype(np.float16)
    bias = rng.normal(size=w.N).astype(np.float16)
    note("epilogue 8192^3 sampled")
    d = run_gemm_ex(A, B, C, bias, 0.5, 2.0)
    rows = np.sort(rng.choice(w.M, 64, replace=False))
    cols = np.sort(rng.choice(w.N, 64, replace=False))
    ref = oracle.gemm_nt_f16_ex(A[rows], B[cols], C[np.ix_(rows, cols)], bias[cols], 0.5, 2.0)
    assert_tolerance(d[np.ix_(rows, cols)], ref, w.K, "epilogue 8192^3", scale=0.5)
