"""Pins of the oracle's FP8 product D = scale * A B^T (A, B in the OCP 8-bit
formats E4M3 or E5M2, fp64 sum, one multiplication by the fp32 scale, one
rounding to fp16).

  f1 decode: every bit pattern of both formats against torch's float8_e4m3fn
     and float8_e5m2 casts, plus the formats' defining constants (largest
     finite, smallest subnormal and normal, one, the NaN and infinity codes);
  f2 brute force on tiny shapes with random finite patterns: the exact
     rational sum times the scale, rounded to fp16 by a nearest-value search;
  f3 integer inputs with a power-of-two scale: the exact integer sum, scaled;
  f4 the scale is applied once, to the exact sum, before the one rounding: a
     scale of 3 on a sum that a rounding of the unscaled sum first would send
     to a tie and the other neighbour, ties, and overflow to infinity;
  f5 mixed formats: A in E5M2 and B in E4M3 against the per-format decode.

Per-channel weight scales (D[m, n] = fp32(a_scale * b_scale[n]) * sum):
  f7 equal column scales reduce to the pinned per-tensor product;
  f8 integer inputs with power-of-two scales that differ per column (and
     M != N, so a scale taken per row would not match): exact;
  f9 brute force on tiny shapes against exact rationals, the column scale
     formed in fp32.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import nearest_f16

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_f1_decode_exhaustive_against_torch():
    import torch
    b = np.arange(256, dtype=np.uint8)
    for e5m2, dt in ((False, torch.float8_e4m3fn), (True, torch.float8_e5m2)):
        d = oracle.fp8_decode(b, e5m2)
        t = torch.from_numpy(b.copy()).view(dt).double().numpy()
        assert np.array_equal(np.isnan(d), np.isnan(t))
        ok = ~np.isnan(t)
        assert np.array_equal(d[ok], t[ok])


def test_f1_decode_defining_constants():
    e4 = oracle.fp8_decode(np.arange(256, dtype=np.uint8), False)
    assert e4[0x38] == 1.0 and e4[0xB8] == -1.0
    assert e4[0x7E] == 448.0 and np.nanmax(e4) == 448.0          # no infinities
    assert e4[0x01] == 2.0 ** -9 and e4[0x08] == 2.0 ** -6
    assert e4[0x07] == 7 * 2.0 ** -9                                # largest subnormal
    assert np.isnan(e4[0x7F]) and np.isnan(e4[0xFF]) and np.isnan(e4).sum() == 2
    e5 = oracle.fp8_decode(np.arange(256, dtype=np.uint8), True)
    assert e5[0x3C] == 1.0 and e5[0x7B] == 57344.0
    assert e5[0x01] == 2.0 ** -16 and e5[0x04] == 2.0 ** -14
    assert e5[0x7C] == np.inf and e5[0xFC] == -np.inf
    assert np.isnan(e5[0x7D:0x80]).all() and np.isnan(e5).sum() == 6
    assert e4[0x80] == 0.0 and np.signbit(e4[0x80]) and e5[0x80] == 0.0
    # monotone over the finite positive codes
    assert np.all(np.diff(e4[:0x7F]) > 0) and np.all(np.diff(e5[:0x7C]) > 0)


def _finite_fp8(seed, shape, e5m2):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    if e5m2:
        bad = (b & 0x7C) == 0x7C
    else:
        bad = (b & 0x7F) == 0x7F
    return np.where(bad, b & 0x83, b).astype(np.uint8)


def _exact_reference(A, B, scale, a_e5m2=False, b_e5m2=False):
    a = [[Fraction(float(v)) for v in r] for r in oracle.fp8_decode(A, a_e5m2)]
    b = [[Fraction(float(v)) for v in r] for r in oracle.fp8_decode(B, b_e5m2)]
    s = Fraction(float(np.float32(scale)))
    out = np.empty((len(a), len(b)), dtype=np.uint16)
    for m in range(len(a)):
        for n in range(len(b)):
            out[m, n] = nearest_f16(s * sum((x * y for x, y in zip(a[m], b[n])), Fraction(0)))
    return out


@pytest.mark.parametrize("e5m2", [False, True])
@pytest.mark.parametrize("K,seed,scale", [(0, 81, 1.0), (1, 82, 0.75), (5, 83, 1.0),
                                          (16, 84, 2.0 ** -7), (33, 85, 0.1)])
def test_f2_brute_force(K, seed, scale, e5m2):
    rng = np.random.default_rng(seed)
    M, N = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    A = _finite_fp8(seed * 10 + 1, (M, K), e5m2)
    B = _finite_fp8(seed * 10 + 2, (N, K), e5m2)
    got = oracle.gemm_nt_fp8(A, B, scale, e5m2, e5m2)
    assert np.array_equal(got, _exact_reference(A, B, scale, e5m2, e5m2))


def _fp8_ints(seed, shape, e5m2):
    """Integers -4..4, exactly representable in both formats."""
    import torch
    v = np.random.default_rng(seed).integers(-4, 5, size=shape).astype(np.float32)
    dt = torch.float8_e5m2 if e5m2 else torch.float8_e4m3fn
    return torch.from_numpy(v).to(dt).view(torch.uint8).numpy()


@pytest.mark.parametrize("e5m2", [False, True])
@pytest.mark.parametrize("M,N,K,scale", [(5, 7, 9, 1.0), (33, 20, 256, 0.5), (8, 3, 96, 4.0)])
def test_f3_integer_exact(M, N, K, scale, e5m2):
    A, B = _fp8_ints(91, (M, K), e5m2), _fp8_ints(92, (N, K), e5m2)
    ai = oracle.fp8_decode(A, e5m2)
    bi = oracle.fp8_decode(B, e5m2)
    assert np.array_equal(ai, np.round(ai)) and np.abs(ai).max() <= 4
    exact = (ai.astype(np.int64) @ bi.astype(np.int64).T) * scale    # power of two: exact
    want = np.array([[nearest_f16(Fraction(float(v))) for v in row] for row in exact], np.uint16)
    assert np.array_equal(oracle.gemm_nt_fp8(A, B, scale, e5m2, e5m2), want)


def _code(x: float, e5m2=False) -> int:
    vals = oracle.fp8_decode(np.arange(256, dtype=np.uint8), e5m2)
    hit = np.flatnonzero(vals == x)
    assert hit.size, f"{x} is not an FP8 value"
    return int(hit[0])


def test_f4_scale_applied_once_after_the_sum():
    # products 1, 2^-11 and 2^-13 (2^-6 times 64, 2^-5 and the subnormal
    # 2^-7): the exact sum S = 1 + 2^-11 + 2^-13 lies above the fp16
    # midpoint of 1 and 1 + 2^-10.
    A = np.array([[_code(2.0 ** -6)] * 3], np.uint8)
    B = np.array([[_code(64.0), _code(2.0 ** -5), _code(2.0 ** -7)]], np.uint8)
    assert int(oracle.gemm_nt_fp8(A, B, 1.0)[0, 0]) == 0x3C01
    # 3S = 3 + 0.9375 * 2^-9 rounds to 3 + 2^-9 (0x4201); rounding S first
    # gives 3 * (1 + 2^-10), a tie that goes to the even 3 + 2^-8 (0x4202)
    assert int(oracle.gemm_nt_fp8(A, B, 3.0)[0, 0]) == 0x4201
    for s in (0.1, 1.0 / 3.0, 1000.0, -2.5):
        S = 1 + Fraction(1, 2048) + Fraction(1, 8192)
        assert int(oracle.gemm_nt_fp8(A, B, s)[0, 0]) == nearest_f16(Fraction(float(np.float32(s))) * S)
    # the exact sum 1 + 2^-11 is a tie and goes to 1; times 2, to 2
    A = np.array([[_code(2.0 ** -6)] * 2], np.uint8)
    B = np.array([[_code(64.0), _code(2.0 ** -5)]], np.uint8)
    assert int(oracle.gemm_nt_fp8(A, B, 1.0)[0, 0]) == 0x3C00
    assert int(oracle.gemm_nt_fp8(A, B, 2.0)[0, 0]) == 0x4000
    # overflow: two products 448 * 448 exceed fp16's range -> infinity,
    # unless the scale brings the sum back
    A = np.array([[0x7E, 0x7E]], np.uint8)
    assert int(oracle.gemm_nt_fp8(A, A, 1.0)[0, 0]) == 0x7C00
    assert int(oracle.gemm_nt_fp8(A, A, -1.0)[0, 0]) == 0xFC00
    assert int(oracle.gemm_nt_fp8(A, A, 2.0 ** -4)[0, 0]) == nearest_f16(Fraction(448 * 448 * 2, 16))


def test_f5_mixed_formats():
    A = _finite_fp8(101, (3, 12), True)
    B = _finite_fp8(102, (4, 12), False)
    got = oracle.gemm_nt_fp8(A, B, 0.25, a_e5m2=True, b_e5m2=False)
    assert np.array_equal(got, _exact_reference(A, B, 0.25, True, False))
    # the same bytes read as the other format give a different product
    assert not np.array_equal(got, oracle.gemm_nt_fp8(A, B, 0.25, False, False))


def test_f6_shape_errors():
    with pytest.raises(ValueError):
        oracle.gemm_nt_fp8(np.zeros((2, 3), np.uint8), np.zeros((2, 4), np.uint8))


def test_f7_column_scales_reduce_to_per_tensor():
    A = _finite_fp8(111, (6, 40), False)
    B = _finite_fp8(112, (9, 40), False)
    for sa, sb in ((0.5, 0.25), (0.1, 3.0), (1.0 / 3.0, 7.0)):
        want = oracle.gemm_nt_fp8(A, B, float(np.float32(sa) * np.float32(sb)))
        got = oracle.gemm_nt_fp8_cs(A, B, sa, np.full(9, sb, np.float32))
        assert np.array_equal(got, want)


@pytest.mark.parametrize("e5m2", [False, True])
def test_f8_column_scales_integer_exact(e5m2):
    M, N, K = 13, 21, 64
    A, B = _fp8_ints(121, (M, K), e5m2), _fp8_ints(122, (N, K), e5m2)
    ai = oracle.fp8_decode(A, e5m2)
    bi = oracle.fp8_decode(B, e5m2)
    sb = (2.0 ** np.random.default_rng(123).integers(-6, 3, N)).astype(np.float32)
    sa = 0.5
    exact = (ai.astype(np.int64) @ bi.astype(np.int64).T) * (sa * sb.astype(np.float64))[None, :]
    want = np.array([[nearest_f16(Fraction(float(v))) for v in row] for row in exact], np.uint16)
    assert np.array_equal(oracle.gemm_nt_fp8_cs(A, B, sa, sb, e5m2, e5m2), want)


@pytest.mark.parametrize("K,seed", [(7, 131), (24, 132)])
def test_f9_column_scales_brute_force(K, seed):
    rng = np.random.default_rng(seed)
    M, N = 3, 4
    A = _finite_fp8(seed * 10 + 1, (M, K), False)
    B = _finite_fp8(seed * 10 + 2, (N, K), True)
    sa = np.float32(rng.uniform(0.01, 2.0))
    sb = rng.uniform(0.01, 2.0, N).astype(np.float32)
    a = [[Fraction(float(v)) for v in r] for r in oracle.fp8_decode(A, False)]
    b = [[Fraction(float(v)) for v in r] for r in oracle.fp8_decode(B, True)]
    want = np.empty((M, N), np.uint16)
    for n in range(N):
        sn = Fraction(float(np.float32(sa * sb[n])))          # the product rounded to fp32
        for m in range(M):
            want[m, n] = nearest_f16(sn * sum((x * y for x, y in zip(a[m], b[n])), Fraction(0)))
    assert np.array_equal(oracle.gemm_nt_fp8_cs(A, B, float(sa), sb, False, True), want)


def test_f9_column_scale_count_checked():
    with pytest.raises(ValueError):
        oracle.gemm_nt_fp8_cs(np.zeros((2, 3), np.uint8), np.zeros((4, 3), np.uint8), 1.0,
                              np.ones(3, np.float32))
