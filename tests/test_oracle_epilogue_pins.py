"""Pins of the oracle's fused epilogue, D = alpha * A B^T + beta * C + bias.

The readings (recorded in the oracle's header): alpha and beta are fp32
values; bias holds one value per output column n; the three terms are formed
and added in fp64 in that order and rounded once to fp16; when beta == 0, C is
not read.  Each pin is independent of the oracle's C code:

  e1 integer inputs with dyadic alpha, beta: the exact rational result (the
     fp16 conversion of a small integer or half-integer is exact);
  e2 brute force on tiny shapes with random fp16 bit patterns and random fp32
     scalars: the same definition evaluated with Python floats in the same
     order, rounded with an independent nearest-fp16 search;
  e3 A = 0: D = beta * C + bias rounded once, by numpy's fp64 -> fp16 cast;
  e4 bias broadcast: with A = 0 and beta = 0 every row of D is the bias row;
  e5 alpha = 1, beta = 0, no bias reduces to the plain product (pinned by its
     own battery), bit for bit; beta = 0 never reads C (NaN there is ignored).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_gemm_18_amd import workloads as wl
from tests.test_oracle_pins import nearest_f16

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _ints(seed, shape, lo=-3, hi=3):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float16)


@pytest.mark.parametrize("alpha,beta", [(2.0, -1.0), (-0.5, 3.0), (1.0, 0.25), (0.0, 1.0),
                                        (-3.0, 0.0)])
@pytest.mark.parametrize("M,N,K", [(7, 9, 13), (33, 17, 64)])
def test_e1_integer_exact(alpha, beta, M, N, K):
    A, B = _ints(1, (M, K)), _ints(2, (N, K))
    C, bias = _ints(3, (M, N), -50, 50), _ints(4, (N,), -20, 20)
    exact = (alpha * (A.astype(np.int64) @ B.astype(np.int64).T)
             + beta * C.astype(np.float64) + bias.astype(np.float64)[None, :])
    # all values are multiples of 1/4 below 2048: exactly representable
    assert np.all(np.abs(exact) < 2048) and np.all(exact * 4 == np.round(exact * 4))
    want = exact.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.gemm_nt_f16_ex(A, B, C, bias, alpha, beta), want)


def _python_fp64_ex(A, B, C, bias, alpha, beta):
    a = A.astype(np.float64).tolist()
    b = B.astype(np.float64).tolist()
    c = C.astype(np.float64).tolist()
    bb = bias.astype(np.float64).tolist()
    al, be = float(np.float32(alpha)), float(np.float32(beta))
    out = np.empty((len(a), len(b)), dtype=np.uint16)
    for m in range(len(a)):
        for n in range(len(b)):
            acc = 0.0
            for x, y in zip(a[m], b[n]):
                acc += x * y
            r = al * acc
            if be != 0.0:
                r = r + be * c[m][n]
            r = r + bb[n]
            out[m, n] = nearest_f16(Fraction(r)) if np.isfinite(r) else (
                0x7C00 if r > 0 else 0xFC00)
    return out


@pytest.mark.parametrize("K", [0, 1, 3, 16])
@pytest.mark.parametrize("seed", [31, 32, 33])
def test_e2_brute_force(K, seed):
    rng = np.random.default_rng(seed)
    M, N = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    A = wl.random_bits(seed * 10 + 1, (M, K))
    B = wl.random_bits(seed * 10 + 2, (N, K))
    C = wl.random_bits(seed * 10 + 3, (M, N))
    bias = wl.random_bits(seed * 10 + 4, (N,))
    alpha, beta = float(rng.normal()), float(rng.normal())
    got = oracle.gemm_nt_f16_ex(A, B, C, bias, alpha, beta)
    assert np.array_equal(got, _python_fp64_ex(A, B, C, bias, alpha, beta))


def test_e3_zero_product_is_scaled_c_plus_bias():
    M, N, K = 20, 30, 40
    A = np.zeros((M, K), np.float16)
    B = wl.uniform_inputs(41, M, N, K)[1]
    C = wl.uniform_inputs(42, M, N, 1)[0][:, :1] * np.ones((1, N), np.float16)
    C = (C * np.arange(1, N + 1, dtype=np.float16)[None, :]).astype(np.float16)
    bias = np.linspace(-3, 3, N).astype(np.float16)
    for beta in (0.3, -1.7, 1.0):
        b32 = float(np.float32(beta))
        want = (b32 * C.astype(np.float64) + bias.astype(np.float64)[None, :]).astype(np.float16)
        got = oracle.gemm_nt_f16_ex(A, B, C, bias, 2.5, beta)
        assert np.array_equal(got, want.view(np.uint16))


def test_e4_bias_is_per_column():
    M, N, K = 6, 11, 5
    A = np.zeros((M, K), np.float16)
    B = np.ones((N, K), np.float16)
    bias = np.arange(N, dtype=np.float16) - 4
    got = oracle.gemm_nt_f16_ex(A, B, None, bias, 1.0, 0.0)
    assert np.array_equal(got, np.tile(bias.view(np.uint16), (M, 1)))


def test_e5_reduces_to_plain_and_ignores_c_at_beta_zero():
    A, B = wl.uniform_inputs(51, 37, 29, 100)
    plain = oracle.gemm_nt_f16(A, B)
    assert np.array_equal(oracle.gemm_nt_f16_ex(A, B), plain)
    C = np.full((37, 29), np.nan, np.float16)
    assert np.array_equal(oracle.gemm_nt_f16_ex(A, B, C, None, 1.0, 0.0), plain)
