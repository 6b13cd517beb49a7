"""Pins for the oracle's fp16-accumulating product, checked against things
other than the oracle itself.

Page "如何用 Croqtile 一步步优化矩阵乘法内核" keeps the running sum in fp16
(the f16 accumulator of its kernels, sections "内核 0：朴素版" and "内核 2：
Hopper TMA + WGMMA").  The oracle's reading: s starts at +0; for each chunk of
64 consecutive k, the chunks aligned to K's end (the first one holds the
K mod 64 leading terms), the chunk's exact sum of products is rounded to fp16
and added to s with an fp16 addition, s <- fp16(s + fp16(chunk sum)), each
rounding to nearest with ties to even; D = s.

  h1  closed form: one 1024 followed by chunks that each sum to 1 climbs by
      1 per chunk and stalls at 2048 (where 2049 is a tie that rounds to
      even), not at the exact sum
  h2  chunk alignment: with K = 65 the first chunk is k = 0 alone
  h3  the chunk is rounded before it is added: a chunk summing to
      0.5 + 2^-12 becomes 0.5 (a tie, to even) and leaves 1024 at 1024 (one
      rounding of 1024.500244 would give 1025); a chunk summing to 2049
      becomes 2048
  h4  one chunk (K <= 64) is the plain product, rounded once (the pinned
      oracle_gemm_nt_f16), except that a sum rounding to -0 gives +0 (the
      fp16 addition +0 + -0); small integers whose partial sums stay within
      2048 give the exact integer result at any K
  h5  brute force: exact rational arithmetic with an independent fp16
      rounding, on tiny shapes with K around the chunk width
  h6  symmetries: D(-A, B) = -D(A, B), D(B, A) = D(A, B)^T
  h7  K = 0 gives +0, and so does a negative sum too small for fp16;
      overflow to infinity and its sign

None of these tests needs a GPU.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_gemm_18_amd import workloads as wl
from tests.test_oracle_pins import _POS_VALS, bits, f16, nearest_f16

W = 64      # products per accumulator update


def _value(b: int) -> Fraction:
    mag = b & 0x7FFF
    assert mag < 0x7C00, "the brute-force inputs keep every partial sum finite"
    v = _POS_VALS[mag]
    return -v if b & 0x8000 else v


def _exact_acc16(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """The definition above in exact rational arithmetic."""
    a = [[Fraction(float(v)) for v in row] for row in A.astype(np.float64)]
    b = [[Fraction(float(v)) for v in row] for row in B.astype(np.float64)]
    K = A.shape[1]
    out = np.empty((len(a), len(b)), dtype=np.uint16)
    for m, ra in enumerate(a):
        for n, rb in enumerate(b):
            s = nearest_f16(Fraction(0))
            k0, length = 0, (K % W) or W
            while k0 < K:
                c = sum((ra[k] * rb[k] for k in range(k0, k0 + length)), Fraction(0))
                s = nearest_f16(_value(s) + _value(nearest_f16(c)))
                k0, length = k0 + length, W
            out[m, n] = s
    return out


def _ones_b(K: int) -> np.ndarray:
    return np.ones((1, K), dtype=np.float16)


# ------------------------------------------------------------------- h1 ---
@pytest.mark.parametrize("chunks,expect", [(1, 1024), (2, 1025), (500, 1523), (1024, 2047),
                                           (1025, 2048), (1100, 2048)])
def test_h1_stall_at_2048(chunks, expect):
    K = W * chunks
    A = np.zeros((1, K), dtype=np.float16)
    A[0, 0] = 1024.0
    A[0, W:] = 2.0 ** -6                  # every later chunk sums to exactly 1
    d = oracle.gemm_nt_f16_acc16(A, _ones_b(K))
    assert float(d.view(np.float16)[0, 0]) == expect
    # the exact sum is 1024 + chunks - 1: a wider running sum would not stall
    if chunks > 1025:
        assert float(oracle.gemm_nt_f16(A, _ones_b(K)).view(np.float16)[0, 0]) > 2048


# ------------------------------------------------------------------- h2 ---
def test_h2_chunks_aligned_to_k_end():
    K = W + 1
    A = np.zeros((1, K), dtype=np.float16)
    A[0, 0], A[0, 1], A[0, W] = 1024.0, 0.5, 0.5
    # chunks {0} and {1..64}: 1024, then 1024 + 1.  Chunks {0..63}, {64}
    # would round 1024.5 and then 1024 + 0.5 to even: 1024.
    assert float(oracle.gemm_nt_f16_acc16(A, _ones_b(K)).view(np.float16)[0, 0]) == 1025.0
    # a chunk width of 64 exactly: with K = 128, k = 64 opens the second chunk
    K = 2 * W
    A = np.zeros((1, K), dtype=np.float16)
    A[0, 0] = 1024.0
    A[0, W - 1] = 0.5
    A[0, W] = 0.5
    # 1024.5 -> 1024 (tie to even), then 1024 + 0.5 -> 1024
    assert float(oracle.gemm_nt_f16_acc16(A, _ones_b(K)).view(np.float16)[0, 0]) == 1024.0


# ------------------------------------------------------------------- h3 ---
def test_h3_chunk_rounded_before_the_add():
    K = 2 * W
    A = np.zeros((1, K), dtype=np.float16)
    A[0, 0] = 1024.0
    A[0, W], A[0, W + 1] = 0.5, 2.0 ** -12
    # the chunk 0.500244140625 rounds to 0.5 (a tie between 0.5 and
    # 0.5 + 2^-11, to even), and 1024 + 0.5 is a tie that stays at 1024; one
    # rounding of 1024 + 0.500244140625 would give 1025
    assert float(oracle.gemm_nt_f16_acc16(A, _ones_b(K)).view(np.float16)[0, 0]) == 1024.0
    # a single chunk summing to 2049 (1024 + 1025) rounds to 2048 (even)
    A = np.zeros((1, W), dtype=np.float16)
    A[0, 0], A[0, 1] = 1024.0, 1025.0
    assert float(oracle.gemm_nt_f16_acc16(A, _ones_b(W)).view(np.float16)[0, 0]) == 2048.0
    # s = 2050, then a chunk of 2049: rounded first it is 2048 and
    # 2050 + 2048 = 4098 is a tie (step 4) that goes to 4096; one rounding of
    # 2050 + 2049 = 4099 would give 4100
    A = np.zeros((1, K), dtype=np.float16)
    A[0, 0], A[0, 1] = 1024.0, 1026.0        # first chunk 2050
    A[0, W], A[0, W + 1] = 1024.0, 1025.0    # second chunk 2049 -> 2048
    assert float(oracle.gemm_nt_f16_acc16(A, _ones_b(K)).view(np.float16)[0, 0]) == 4096.0
    # each product is rounded with the rest of its chunk, not on its own:
    # 64 products of 2^-6 on top of 1024 give 1025, one at a time they vanish
    A = np.zeros((1, K), dtype=np.float16)
    A[0, 0] = 1024.0
    A[0, W:] = 2.0 ** -6
    assert float(oracle.gemm_nt_f16_acc16(A, _ones_b(K)).view(np.float16)[0, 0]) == 1025.0


# ------------------------------------------------------------------- h4 ---
@pytest.mark.parametrize("K", [1, 7, 33, 63, 64])
@pytest.mark.parametrize("seed", [41, 42])
def test_h4_one_chunk_is_the_plain_product(K, seed):
    rng = np.random.default_rng(seed)
    M, N = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    A = wl.random_bits(seed * 100 + K, (M, K), finite_max=64.0)
    B = wl.random_bits(seed * 100 + K + 50, (N, K), finite_max=64.0)
    plain = oracle.gemm_nt_f16(A, B)
    plain[plain == 0x8000] = 0
    assert np.array_equal(oracle.gemm_nt_f16_acc16(A, B), plain)


@pytest.mark.parametrize("K", [65, 129, 200, 1000])
def test_h4_small_integers_are_exact(K):
    rng = np.random.default_rng(K)
    A = rng.integers(-1, 2, size=(5, K)).astype(np.float16)
    B = rng.integers(-1, 2, size=(6, K)).astype(np.float16)
    exact = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.abs(exact).max() <= 2048 and K <= 2048      # every partial sum too
    d = oracle.gemm_nt_f16_acc16(A, B).view(np.float16).astype(np.float64)
    assert np.array_equal(d, exact.astype(np.float64))


# ------------------------------------------------------------------- h5 ---
@pytest.mark.parametrize("K", [1, 63, 64, 65, 127, 128, 130, 200])
@pytest.mark.parametrize("seed", [51, 52])
def test_h5_brute_force_exact(K, seed):
    # inputs in {0} U +-[2^-8, 4]: every chunk sum and every s + chunk sum is
    # exact in fp64, so the oracle must equal the exact definition
    rng = np.random.default_rng(seed)
    M, N = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    A = wl.random_bits(seed * 1000 + K, (M, K), finite_max=4.0).copy()
    B = wl.random_bits(seed * 1000 + K + 500, (N, K), finite_max=4.0).copy()
    A[np.abs(A.astype(np.float64)) < 2.0 ** -8] = 0
    B[np.abs(B.astype(np.float64)) < 2.0 ** -8] = 0
    assert np.array_equal(oracle.gemm_nt_f16_acc16(A, B), _exact_acc16(A, B))


def test_h5_brute_force_large_sums():
    # integers 3..9 over 1000 terms (16 chunks): chunk sums around 2300,
    # above 2048 where odd integers round, and partial sums up to ~36000,
    # where the fp16 running sum has a step of 2 to 32 and every update rounds
    rng = np.random.default_rng(55)
    K = 1000
    A = rng.integers(3, 10, size=(4, K)).astype(np.float16)
    B = rng.integers(3, 10, size=(4, K)).astype(np.float16)
    got = oracle.gemm_nt_f16_acc16(A, B)
    assert np.array_equal(got, _exact_acc16(A, B))
    # and it is not the once-rounded exact sum everywhere
    assert not np.array_equal(got, oracle.gemm_nt_f16(A, B))


# ------------------------------------------------------------------- h6 ---
def test_h6_symmetries():
    A = wl.random_bits(61, (7, 300), finite_max=8.0)
    B = wl.random_bits(62, (5, 300), finite_max=8.0)
    d = oracle.gemm_nt_f16_acc16(A, B)
    neg = oracle.gemm_nt_f16_acc16(-A, B)
    nz = (d & 0x7FFF) != 0
    assert np.array_equal(neg[nz], d[nz] ^ 0x8000)
    assert np.array_equal(oracle.gemm_nt_f16_acc16(B, A), d.T)


# ------------------------------------------------------------------- h7 ---
def test_h7_empty_overflow_and_sign():
    z = oracle.gemm_nt_f16_acc16(np.zeros((3, 0), np.float16), np.zeros((2, 0), np.float16))
    assert z.shape == (3, 2) and np.all(z == 0)
    # -2^-26 rounds to -0 as a chunk; +0 + -0 is +0 (the plain product is -0)
    A = np.full((1, 1), -(2.0 ** -12), dtype=np.float16)
    B = np.full((1, 1), 2.0 ** -14, dtype=np.float16)
    assert oracle.gemm_nt_f16(A, B)[0, 0] == 0x8000
    assert oracle.gemm_nt_f16_acc16(A, B)[0, 0] == 0
    A = np.full((2, 256), 16.0, dtype=np.float16)
    # chunks of 16384: 16384, 32768, 49152, then 65536 -> infinity
    assert np.all(oracle.gemm_nt_f16_acc16(A, A) == 0x7C00)
    assert np.all(oracle.gemm_nt_f16_acc16(A, -A) == 0xFC00)
    # three chunks stay finite
    A3 = np.full((1, 192), 16.0, dtype=np.float16)
    assert float(oracle.gemm_nt_f16_acc16(A3, A3).view(np.float16)[0, 0]) == 49152.0


def test_entries_agree_with_full():
    A = wl.random_bits(71, (40, 333), finite_max=2.0)
    B = wl.random_bits(72, (30, 333), finite_max=2.0)
    full = oracle.gemm_nt_f16_acc16(A, B)
    rows = np.array([0, 39, 17, 5])
    cols = np.array([29, 0, 11, 5])
    assert np.array_equal(oracle.gemm_nt_f16_acc16_entries(A, B, rows, cols), full[rows, cols])
    with pytest.raises(IndexError):
        oracle.gemm_nt_f16_acc16_entries(A, B, [40], [0])


def test_f16_helpers_are_the_plain_pins_helpers():
    # the rounding used above is the one pinned exhaustively in p1
    assert nearest_f16(Fraction(2049)) == int(bits(f16(2048.0))[()])
