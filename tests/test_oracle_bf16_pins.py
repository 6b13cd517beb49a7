"""Pins of the oracle's bfloat16 product D = A B^T (bfloat16 storage, fp64
sum, one rounding to bfloat16 with round to nearest, ties to even).

  b1 decode: every bit pattern against torch's bfloat16 -> float64 cast;
  b2 encode: round trip of every finite pattern, every midpoint between
     neighbours (ties to the even pattern), midpoints +- one fp64 ulp, the
     overflow threshold, and random values, against an independent
     nearest-bfloat16 search over exact rationals;
  b3 brute force on tiny shapes with random bit patterns: a Python-float
     sequential sum rounded by that search;
  b4 integer inputs: the exact integer sum rounded by that search (sums above
     256 are rounded: bfloat16 has 8 significant bits).
"""
from __future__ import annotations

import bisect
from fractions import Fraction

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

_POS = np.arange(0x7F80, dtype=np.uint32)                      # +0 .. largest finite
_POS_VALS = [Fraction(float(v)) for v in (_POS << 16).astype(np.uint32).view(np.float32)]
_OVERFLOW = (2 - Fraction(1, 256)) * Fraction(2) ** 127        # midpoint to 2^128


def nearest_bf16(x: Fraction) -> int:
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a >= _OVERFLOW:
        return sign | 0x7F80
    i = bisect.bisect_left(_POS_VALS, a)
    if _POS_VALS[i] == a:
        return sign | i
    lo, hi = i - 1, i
    dlo, dhi = a - _POS_VALS[lo], _POS_VALS[hi] - a
    pick = lo if dlo < dhi else hi if dhi < dlo else (lo if lo % 2 == 0 else hi)
    return sign | pick


def _random_bf16_bits(seed, shape):
    """Finite bfloat16 patterns, subnormals and extremes included."""
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 0x10000, size=shape, dtype=np.uint32).astype(np.uint16)
    return np.where((b & 0x7F80) == 0x7F80, b & 0x807F, b).astype(np.uint16)


def test_b1_decode_exhaustive():
    import torch
    b = np.arange(65536, dtype=np.uint16)
    d = oracle.bf16_decode(b)
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(d), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(d[ok], t[ok])


def test_b2_encode_roundtrip_and_midpoints():
    b = np.arange(0x7F80, dtype=np.uint16)                      # finite positives
    v = oracle.bf16_decode(b)
    assert np.array_equal(oracle.bf16_encode(v), b)
    assert np.array_equal(oracle.bf16_encode(-v), b | 0x8000)
    mids = [(_POS_VALS[i] + _POS_VALS[i + 1]) / 2 for i in range(0, 0x7F7F, 97)]
    for m in mids:
        x = float(m)
        assert Fraction(x) == m                                # exact in fp64
        assert oracle.bf16_encode(np.array([x]))[0] == nearest_bf16(m)
        for y in (np.nextafter(x, 0.0), np.nextafter(x, np.inf)):
            assert oracle.bf16_encode(np.array([y]))[0] == nearest_bf16(Fraction(y))


def test_b2_encode_overflow_and_random():
    thr = float(_OVERFLOW)
    got = oracle.bf16_encode(np.array([thr, np.nextafter(thr, 0.0), -thr, np.inf, -np.inf]))
    assert got.tolist() == [0x7F80, 0x7F7F, 0xFF80, 0x7F80, 0xFF80]
    rng = np.random.default_rng(5)
    x = rng.normal(size=2000) * np.exp2(rng.integers(-140, 128, size=2000))
    want = [nearest_bf16(Fraction(float(v))) for v in x]
    assert oracle.bf16_encode(x).tolist() == want


def _python_ref(A, B):
    a = oracle.bf16_decode(A).tolist()
    b = oracle.bf16_decode(B).tolist()
    out = np.empty((len(a), len(b)), dtype=np.uint16)
    for m in range(len(a)):
        for n in range(len(b)):
            acc = 0.0
            for x, y in zip(a[m], b[n]):
                acc += x * y
            out[m, n] = nearest_bf16(Fraction(acc)) if np.isfinite(acc) else (
                0x7F80 if acc > 0 else 0xFF80)
    return out


@pytest.mark.parametrize("K", [0, 1, 3, 8, 17])
@pytest.mark.parametrize("seed", [61, 62])
def test_b3_brute_force(K, seed):
    rng = np.random.default_rng(seed)
    M, N = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    A = _random_bf16_bits(seed * 10 + 1, (M, K))
    B = _random_bf16_bits(seed * 10 + 2, (N, K))
    assert np.array_equal(oracle.gemm_nt_bf16(A, B), _python_ref(A, B))


def _bf16_ints(seed, shape):
    vals = np.random.default_rng(seed).integers(-3, 4, size=shape).astype(np.float32)
    return (vals.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("M,N,K", [(5, 7, 9), (33, 20, 300)])
def test_b4_integer_exact_then_rounded(M, N, K):
    A, B = _bf16_ints(71, (M, K)), _bf16_ints(72, (N, K))
    ai = oracle.bf16_decode(A).astype(np.int64)
    bi = oracle.bf16_decode(B).astype(np.int64)
    exact = ai @ bi.T
    want = np.array([[nearest_bf16(Fraction(int(v))) for v in row] for row in exact], np.uint16)
    assert np.array_equal(oracle.gemm_nt_bf16(A, B), want)
    rows = np.array([0, M - 1, 2]); cols = np.array([N - 1, 0, 3])
    assert np.array_equal(oracle.gemm_nt_bf16_entries(A, B, rows, cols), want[rows, cols])


def _bf(x: float) -> int:
    return nearest_bf16(Fraction(x))


def test_b5_ties_and_double_rounding():
    # bfloat16 has 7 fraction bits: 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7.
    def run(a, b):
        A = np.array([[_bf(v) for v in a]], np.uint16)
        B = np.array([[_bf(v) for v in b]], np.uint16)
        return int(oracle.gemm_nt_bf16(A, B)[0, 0])
    assert run([1.0, 2.0 ** -8], [1.0, 1.0]) == 0x3F80                   # tie -> even (1.0)
    assert run([1.0 + 2.0 ** -7, 2.0 ** -8], [1.0, 1.0]) == 0x3F82       # tie -> even (1 + 2^-6)
    # exact 1 + 2^-8 + 2^-40 lies above the midpoint: rounds up directly,
    # but a detour through fp32 (23 fraction bits) drops 2^-40 and ties down
    assert run([1.0, 2.0 ** -8, 2.0 ** -20], [1.0, 1.0, 2.0 ** -20]) == 0x3F81
