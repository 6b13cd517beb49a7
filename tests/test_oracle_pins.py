"""Pins for the CPU oracle, checked against things other than the oracle itself.

The oracle computes D[m,n] = sum_k A[m,k] * B[n,k] (page "构建 Tiled GEMM",
section "GEMM"), fp16 in, fp64 sum, one rounding to fp16.  The pages print
no matrices or output values, so these pins come from the IEEE binary16
definition, exact rational arithmetic, closed forms and invariants:

  p1  fp16 codec, exhaustive, against numpy's independent conversion
  p2  brute force on tiny shapes: (a) an independent Python evaluation of the
      same definition, (b) the exact rational result rounded once
  p3  identity and permutation operands (layout: D = A B^T, not A B)
  p4  integer {-2..2} inputs against exact integer sums, with ragged tails
  p5  closed forms: all-ones, rank-1
  p6  invariants: D(A,B) = D(B,A)^T, K-split additivity on integers
  p7  ties and double rounding (one rounding from fp64, never via fp32)
  p8  subnormal inputs, overflow to infinity, signed zero, K = 0

None of these tests needs a GPU.
"""
from __future__ import annotations

import bisect
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_gemm_18_amd import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# --------------------------------------------------------------------------
# An independent fp16 rounding: nearest neighbour among all finite fp16
# values (taken from numpy's decode), exact rational comparisons, ties to the
# pattern with an even last bit, and |x| >= 65520 (half-way between 65504 and
# 2^16) to infinity.
_POS_BITS = np.arange(0x7C00, dtype=np.uint16)
_POS_VALS = [Fraction(float(v)) for v in _POS_BITS.view(np.float16).astype(np.float64)]


def nearest_f16(x: Fraction) -> int:
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a >= 65520:
        return sign | 0x7C00
    i = bisect.bisect_left(_POS_VALS, a)
    if _POS_VALS[i] == a:
        return sign | i
    lo, hi = i - 1, i
    dlo, dhi = a - _POS_VALS[lo], _POS_VALS[hi] - a
    if dlo < dhi:
        pick = lo
    elif dhi < dlo:
        pick = hi
    else:
        pick = lo if lo % 2 == 0 else hi
    return sign | pick


def f16(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float16).view(np.uint16)


# ------------------------------------------------------------------- p1 ---
def test_p1_decode_exhaustive():
    allbits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(allbits)
    ref = allbits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zeros too
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_p1_encode_roundtrip_exhaustive():
    allbits = np.arange(65536, dtype=np.uint16)
    vals = allbits.view(np.float16).astype(np.float64)
    fin = ~np.isnan(vals)
    assert np.array_equal(oracle.encode(vals[fin]), allbits[fin])
    assert np.all(oracle.encode(vals[~fin]) == 0x7E00)


def test_p1_encode_midpoints_and_neighbours():
    # every pair of consecutive non-negative finite fp16 values
    b = np.arange(0x7BFF, dtype=np.uint16)
    lo = b.view(np.float16).astype(np.float64)
    hi = (b + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2                          # exact in fp64
    even = np.where(b % 2 == 0, b, b + 1).astype(np.uint16)
    assert np.array_equal(oracle.encode(mid), even)
    assert np.array_equal(oracle.encode(-mid), even | 0x8000)
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    assert np.array_equal(oracle.encode(below), b)
    assert np.array_equal(oracle.encode(above), (b + 1).astype(np.uint16))
    # numpy's conversion agrees on all of them
    for v in (mid, below, above, -mid):
        assert np.array_equal(oracle.encode(v), v.astype(np.float16).view(np.uint16))


def test_p1_encode_overflow_and_random():
    assert oracle.encode(np.array([65504.0 + 16.0]))[0] == 0x7C00       # tie -> inf
    assert oracle.encode(np.array([65504.0 + 15.99]))[0] == 0x7BFF
    assert oracle.encode(np.array([-65520.0]))[0] == 0xFC00
    assert oracle.encode(np.array([1e300, -1e300, np.inf, -np.inf])).tolist() == [
        0x7C00, 0xFC00, 0x7C00, 0xFC00]
    assert oracle.encode(np.array([2.0 ** -25]))[0] == 0x0000            # tie -> even (0)
    assert oracle.encode(np.array([3 * 2.0 ** -26]))[0] == 0x0001        # above half
    assert oracle.encode(np.array([-(2.0 ** -26)]))[0] == 0x8000         # -> -0
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200_000) * np.exp2(rng.uniform(-30, 18, 200_000))
    assert np.array_equal(oracle.encode(x), x.astype(np.float16).view(np.uint16))


# ------------------------------------------------------------------- p2 ---
def _python_fp64_reference(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Same definition, written independently: Python floats, sequential."""
    a = A.astype(np.float64).tolist()
    b = B.astype(np.float64).tolist()
    M, N = len(a), len(b)
    out = np.empty((M, N), dtype=np.uint16)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for x, y in zip(a[m], b[n]):
                acc += x * y
            out[m, n] = nearest_f16(Fraction(acc))
    return out


def _exact_reference(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """The exact rational sum, rounded once."""
    a = [[Fraction(float(v)) for v in row] for row in A.astype(np.float64)]
    b = [[Fraction(float(v)) for v in row] for row in B.astype(np.float64)]
    out = np.empty((len(a), len(b)), dtype=np.uint16)
    for m, ra in enumerate(a):
        for n, rb in enumerate(b):
            out[m, n] = nearest_f16(sum((x * y for x, y in zip(ra, rb)), Fraction(0)))
    return out


@pytest.mark.parametrize("K", [0, 1, 2, 3, 7, 16, 17])
@pytest.mark.parametrize("seed", [11, 12, 13])
def test_p2a_brute_force_any_finite(K, seed):
    rng = np.random.default_rng(seed)
    M, N = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    A = wl.random_bits(seed * 100 + 1, (M, K))
    B = wl.random_bits(seed * 100 + 2, (N, K))
    assert np.array_equal(oracle.gemm_nt_f16(A, B), _python_fp64_reference(A, B))


@pytest.mark.parametrize("K", [1, 2, 5, 16, 33, 64])
@pytest.mark.parametrize("seed", [21, 22])
def test_p2b_exact_rational(K, seed):
    # inputs in {0} U +-[2^-8, 4]: fp64 sums of at most 64 such products are
    # exact (multiples of 2^-36 below 2^10), so the oracle must equal the
    # exact result rounded once.
    rng = np.random.default_rng(seed)
    M, N = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    A = wl.random_bits(seed * 100 + 3, (M, K), finite_max=4.0).copy()
    B = wl.random_bits(seed * 100 + 4, (N, K), finite_max=4.0).copy()
    A[np.abs(A.astype(np.float64)) < 2.0 ** -8] = 0
    B[np.abs(B.astype(np.float64)) < 2.0 ** -8] = 0
    assert np.array_equal(oracle.gemm_nt_f16(A, B), _exact_reference(A, B))


# ------------------------------------------------------------------- p3 ---
def test_p3_identity_and_permutation():
    rng = np.random.default_rng(31)
    K = 37
    B = f16(rng.uniform(-1, 1, (23, K)))
    A = f16(rng.uniform(-1, 1, (19, K)))
    B[B == 0] = 0.5         # no zeros: avoids +-0 ambiguity in bitwise compare
    A[A == 0] = 0.5
    eye = np.eye(K, dtype=np.float16)
    assert np.array_equal(oracle.gemm_nt_f16(eye, B), bits(B.T))        # A = I -> B^T
    assert np.array_equal(oracle.gemm_nt_f16(A, eye), bits(A))          # B = I -> A
    perm = rng.permutation(K)
    P = np.zeros((K, K), dtype=np.float16)
    P[np.arange(K), perm] = 1                                            # P[m, perm[m]] = 1
    D = oracle.gemm_nt_f16(P, B)                                         # D[m,n] = B[n, perm[m]]
    assert np.array_equal(D, bits(B[:, perm].T))
    # a non-square permutation of rows of B picks columns of D
    D2 = oracle.gemm_nt_f16(A, P)                                        # D[m,n] = A[m, perm[n]]
    assert np.array_equal(D2, bits(A[:, perm]))


# ------------------------------------------------------------------- p4 ---
@pytest.mark.parametrize("shape", [(1, 1, 1), (5, 3, 2), (33, 65, 129), (130, 70, 67),
                                   (128, 128, 64), (257, 129, 1000), (64, 300, 2050)])
def test_p4_integer_exact(shape):
    M, N, K = shape
    A, B = wl.integer_free(41 + M, M, N, K)
    exact = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.abs(exact).max() <= 2048
    assert np.array_equal(oracle.gemm_nt_f16(A, B), bits(exact.astype(np.float64)))


@pytest.mark.parametrize("name", ["tile_128x128x64", "square_1024"])
def test_p4_integer_workloads(name):
    w = wl.WORKLOADS[name]
    A, B = wl.integer_inputs(w)
    exact = A.astype(np.float64) @ B.astype(np.float64).T     # integers: exact in fp64
    assert np.abs(exact).max() <= 2048
    assert np.array_equal(oracle.gemm_nt_f16(A, B), bits(exact))


# ------------------------------------------------------------------- p5 ---
@pytest.mark.parametrize("K", [64, 1024, 2050, 8192])
def test_p5_all_ones(K):
    A = np.ones((3, K), dtype=np.float16)
    B = np.ones((4, K), dtype=np.float16)
    assert np.all(oracle.gemm_nt_f16(A, B) == bits(np.float64(K)))


def test_p5_rank_one():
    rng = np.random.default_rng(51)
    K = 300
    a = rng.integers(-3, 4, 17)
    b = rng.integers(-3, 4, 29)
    A = np.repeat(a[:, None], K, axis=1).astype(np.float16)
    B = np.repeat(b[:, None], K, axis=1).astype(np.float16)
    expect = (K * np.outer(a, b)).astype(np.float64)
    assert np.array_equal(oracle.gemm_nt_f16(A, B), bits(expect))


# ------------------------------------------------------------------- p6 ---
def test_p6_transpose_symmetry():
    A, B = wl.uniform_inputs(61, 37, 53, 211)
    assert np.array_equal(oracle.gemm_nt_f16(A, B), oracle.gemm_nt_f16(B, A).T)


def test_p6_k_split_additivity():
    A, B = wl.integer_free(62, 40, 50, 300)
    D = oracle.decode(oracle.gemm_nt_f16(A, B))
    D1 = oracle.decode(oracle.gemm_nt_f16(A[:, :113], B[:, :113]))
    D2 = oracle.decode(oracle.gemm_nt_f16(A[:, 113:], B[:, 113:]))
    assert np.array_equal(D, D1 + D2)


def test_entries_agree_with_full():
    A, B = wl.uniform_inputs(63, 70, 90, 129)
    D = oracle.gemm_nt_f16(A, B)
    rows = np.array([0, 69, 35, 1, 69])
    cols = np.array([0, 89, 44, 88, 0])
    assert np.array_equal(oracle.gemm_nt_f16_entries(A, B, rows, cols), D[rows, cols])
    with pytest.raises(IndexError):
        oracle.gemm_nt_f16_entries(A, B, [70], [0])


# ------------------------------------------------------------------- p7 ---
def test_p7_ties_and_double_rounding():
    one = 1.0
    # 1 + 2^-11 is exactly half-way between 0x3C00 and 0x3C01 -> even 0x3C00
    assert oracle.gemm_nt_f16(f16([[one, 2 ** -11]]), f16([[1, 1]]))[0, 0] == 0x3C00
    # (1 + 2^-10) + 2^-11 is half-way between 0x3C01 and 0x3C02 -> even 0x3C02
    assert oracle.gemm_nt_f16(f16([[1 + 2 ** -10, 2 ** -11]]), f16([[1, 1]]))[0, 0] == 0x3C02
    # 1 + 2^-11 + 2^-40: above the tie, rounds up to 0x3C01 when rounded once;
    # a detour through fp32 would make it the tie and give 0x3C00.
    A = f16([[1, 2 ** -11, 2 ** -20]])
    B = f16([[1, 1, 2 ** -20]])
    assert oracle.gemm_nt_f16(A, B)[0, 0] == 0x3C01
    via_f32 = np.float32(1 + 2 ** -11 + 2 ** -40)
    assert bits(np.float16(via_f32)) == 0x3C00      # what the wrong path would give


# ------------------------------------------------------------------- p8 ---
@pytest.mark.parametrize("K", [1, 7, 64, 1024])
def test_p8_subnormal_inputs(K):
    A = np.full((2, K), 2.0 ** -24, dtype=np.float16)       # 0x0001, smallest subnormal
    assert bits(A)[0, 0] == 0x0001
    B = np.full((3, K), 1024.0, dtype=np.float16)
    D = oracle.gemm_nt_f16(A, B)
    assert np.all(D == bits(np.float64(K) * 2.0 ** -14))    # K * 2^-14, exact, nonzero


def test_p8_overflow_and_signed_zero_and_empty():
    A = np.full((2, 256), 16.0, dtype=np.float16)
    assert np.all(oracle.gemm_nt_f16(A, A) == 0x7C00)        # 65536 -> +inf
    assert np.all(oracle.gemm_nt_f16(A, -A) == 0xFC00)
    negz = np.full((2, 5), -0.0, dtype=np.float16)
    pos = np.ones((3, 5), dtype=np.float16)
    assert np.all(oracle.gemm_nt_f16(negz, pos) == 0x0000)   # sum of -0 from +0 is +0
    assert oracle.gemm_nt_f16(np.zeros((4, 0), np.float16), np.zeros((3, 0), np.float16)).tolist() == [[0] * 3] * 4
    assert oracle.gemm_nt_f16(np.zeros((0, 5), np.float16), pos).shape == (0, 3)
