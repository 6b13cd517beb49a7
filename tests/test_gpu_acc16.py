"""GPU parity of gemm_nt_f16_acc16 (fp16 running sum) against the oracle.

The definition (the f16 accumulator of page "如何用 Croqtile 一步步优化矩阵乘法
内核", sections "内核 0：朴素版" and "内核 2：Hopper TMA + WGMMA"; rounding points
as the oracle states them): s starts at +0, and for each chunk of 64
consecutive k, aligned to K's end, s <- fp16(s + fp16(chunk sum)).

Where the kernel's fp32 chunk sums are exact the two sides round the same
values at the same points, so the result must match bit for bit: integer
inputs (chunk sums above 2048 and running sums up to ~20000, so both
roundings act) and "coarse" inputs, multiples of 2^-6 in [-2, 2], whose
chunk sums have at most 20 significant bits.  Every case first asks the
library which kernel it takes and asserts the one it targets.

For general random inputs the fp32 chunk sum may differ from the exact one
by at most 2^-18 times the chunk's sum of |products| (64 fp32 additions), so
a chunk's rounding to fp16 and the following addition can each land one
fp16 step apart; the difference of the two running sums is then bounded by
    sum_j [ulp(|c_j|) + 2^-18 sum_{k in j} |a_k b_k| + ulp(1.25 P)]
with c_j the exact chunk sums, P = sum_j |c_j| and ulp(x) <= 2^-10 x + 2^-24
the fp16 step at x.  The test checks that bound and that nearly every entry
is bit-identical anyway.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from dense_gemm_18_amd import binding
from dense_gemm_18_amd import workloads as wl
from tests.gpu_util import assert_bitexact, note, run_gemm

pytestmark = pytest.mark.gpu

ALIGNED = 1 << 20          # a 16-byte aligned stand-in address (never dereferenced)
W = 64


@pytest.fixture(scope="module", autouse=True)
def _library_present():
    assert binding.library_path().exists(), "libgemm18.so not built"


def _kernel(M, N, K, a_off=0, b_off=0):
    return binding.gemm_nt_f16_acc16_kernel(ALIGNED + 2 * a_off, 2 * ALIGNED + 2 * b_off, M, N, K)


def _big_integers(seed, M, N, K):
    # entries 4..8: chunk sums ~2300 (odd ones above 2048 round), running
    # sums up to ~36 per k
    rng = np.random.default_rng(seed)
    A = rng.integers(4, 9, size=(M, K)).astype(np.float16)
    B = rng.integers(4, 9, size=(N, K)).astype(np.float16)
    return A, B


def _run(A, B, **kw):
    return run_gemm(A, B, acc16=True, **kw)


# (M, N, K, a_off, b_off, tile, load bytes): the 256 x 256 (8 waves), 128 x 128
# (four stages with at most 256 tiles, two beyond: 2300 x 2200) and 64 x 64
# tiles with direct loads, also at rows not 16-byte aligned (odd K, K % 8
# != 0, 2-byte aligned operands; 2900 x 4100 x 521), and the register-staged
# 128 x 128 and 64 x 64 kernels (K < 8; skinny shapes with such rows)
CASES = [(2900, 4100, 512, 0, 0, 256, 16), (2900, 4100, 520, 0, 0, 256, 16),
         (1000, 1100, 576, 0, 0, 128, 16), (700, 900, 200, 0, 0, 128, 16),
         (2300, 2200, 264, 0, 0, 128, 16),
         (64, 3000, 448, 0, 0, 64, 16), (3000, 40, 200, 0, 0, 64, 16),
         (1000, 1100, 577, 0, 0, 128, 16), (700, 900, 202, 0, 0, 128, 16),
         (1000, 1100, 512, 1, 0, 128, 16), (700, 900, 200, 0, 3, 128, 16),
         (2900, 4100, 521, 0, 0, 256, 16), (1000, 1100, 5, 0, 0, 128, 1),
         (64, 3000, 449, 0, 0, 64, 1), (3000, 40, 130, 2, 0, 64, 1)]


@pytest.mark.parametrize("M,N,K,a_off,b_off,bm,lb", CASES)
def test_acc16_integer(M, N, K, a_off, b_off, bm, lb):
    tbm, tbn, tlb = _kernel(M, N, K, a_off, b_off)
    assert (tbm, tlb) == (bm, lb), (tbm, tbn, tlb)
    A, B = _big_integers(17000 + K + a_off, M, N, K)
    note(f"acc16 integer {M}x{N}x{K} a+{a_off} b+{b_off} tile {tbm}x{tbn} load {tlb}")
    d = _run(A, B, a_off=a_off, b_off=b_off)
    ref = oracle.gemm_nt_f16_acc16(A, B)
    if K >= 128:
        assert oracle.decode(ref).max() > 4096      # the fp16 running sum rounds
    assert_bitexact(d, ref, f"acc16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,a_off,b_off,bm,lb", CASES[::2])
def test_acc16_coarse_random(M, N, K, a_off, b_off, bm, lb):
    assert _kernel(M, N, K, a_off, b_off)[0::2] == (bm, lb)
    A, B = wl.coarse_uniform(17500 + K, M, N, K)
    note(f"acc16 coarse {M}x{N}x{K} a+{a_off} b+{b_off}")
    assert_bitexact(_run(A, B, a_off=a_off, b_off=b_off), oracle.gemm_nt_f16_acc16(A, B),
                    f"acc16 coarse {M}x{N}x{K}")


def _bound(A, B):
    """The per-entry bound of the module docstring, in fp64."""
    a = A.astype(np.float64)
    b = B.astype(np.float64)
    K = a.shape[1]
    first = K % W or W
    edges = [0] + list(range(first, K + 1, W)) if K else [0]
    tol = np.zeros((a.shape[0], b.shape[0]))
    P = np.zeros_like(tol)
    for k0, k1 in zip(edges[:-1], edges[1:]):
        c = np.abs(a[:, k0:k1] @ b[:, k0:k1].T)
        s = np.abs(a[:, k0:k1]) @ np.abs(b[:, k0:k1]).T
        tol += 2.0 ** -10 * c + 2.0 ** -24 + 2.0 ** -18 * s
        P += c
    nk = len(edges) - 1
    return tol + nk * (2.0 ** -10 * 1.25 * P + 2.0 ** -24)


@pytest.mark.parametrize("M,N,K,a_off", [(2900, 4100, 512, 0), (1000, 1100, 1000, 0),
                                         (700, 900, 1001, 0), (64, 3000, 2048, 1)])
def test_acc16_uniform_random(M, N, K, a_off):
    A, B = wl.uniform_inputs(18000 + K, M, N, K)
    note(f"acc16 uniform {M}x{N}x{K} a+{a_off}")
    d = oracle.decode(_run(A, B, a_off=a_off))
    ref = oracle.decode(oracle.gemm_nt_f16_acc16(A, B))
    err = np.abs(d - ref)
    tol = _bound(A, B)
    bad = np.flatnonzero(~(err <= tol))
    assert bad.size == 0, f"{bad.size} entries outside the bound, first {bad[:5]}"
    same = np.count_nonzero(err == 0) / err.size
    print(f"acc16 uniform {M}x{N}x{K}: {same:.4f} of entries bit-identical, "
          f"max error {err.max():.3g}, max bound {tol.max():.3g}")
    assert same >= 0.99


@pytest.mark.parametrize("K", list(range(1, 131)))
def test_acc16_every_k_tail(K):
    A, B = _big_integers(19000 + K, 67, 45, K)
    note(f"acc16 K tail K={K}")
    assert_bitexact(_run(A, B), oracle.gemm_nt_f16_acc16(A, B), f"acc16 K={K}")


@pytest.mark.parametrize("M,N", [(1, 1), (1, 300), (300, 1), (63, 65), (65, 63), (129, 257),
                                 (257, 129), (513, 1031)])
def test_acc16_mn_sweep(M, N):
    A, B = _big_integers(19500 + M * 7 + N, M, N, 136)
    note(f"acc16 MN sweep {M}x{N}x136")
    assert_bitexact(_run(A, B), oracle.gemm_nt_f16_acc16(A, B), f"acc16 {M}x{N}")
    assert_bitexact(_run(A, B, d_off=4), oracle.gemm_nt_f16_acc16(A, B), f"acc16 {M}x{N} d+4")


def test_acc16_headline_sampled():
    # the 8192^3 workload's shape through the 256 x 256 tile: coarse inputs,
    # 4096 seeded entries plus full rows and columns at tile edges
    w = wl.WORKLOADS[wl.HEADLINE]
    assert _kernel(w.M, w.N, w.K) == (256, 256, 16)
    A, B = wl.coarse_uniform(w.seeds[0] + 100, w.M, w.N, w.K)
    note(f"acc16 {w.name} coarse (sampled + tile-edge rows/cols)")
    d = _run(A, B)
    rows, cols = wl.sample_indices(w, 4096)
    er, ec = wl.edge_lines(w.M, 256), wl.edge_lines(w.N, 256)
    rr = np.concatenate([rows, np.repeat(er, w.N), np.tile(np.arange(w.M), ec.size)])
    cc = np.concatenate([cols, np.tile(np.arange(w.N), er.size), np.repeat(ec, w.M)])
    ref = oracle.gemm_nt_f16_acc16_entries(A, B, rr, cc)
    assert_bitexact(d[rr, cc], ref, f"acc16 {w.name} sampled")


def test_acc16_agrees_with_fp32_path_below_2048():
    # small integers: every partial sum is an integer of at most 2048, so the
    # fp16 and fp32 running sums are both exact
    A, B = wl.integer_free(19900, 1000, 1100, 1000, -1, 1)
    note("acc16 vs fp32 path, |sums| <= 1000")
    d16 = _run(A, B)
    assert_bitexact(d16, run_gemm(A, B), "acc16 vs gemm_nt_f16")
    assert_bitexact(d16, oracle.gemm_nt_f16(A, B), "acc16 vs exact")


def test_acc16_edges():
    note("acc16 K=0")
    d = _run(np.zeros((70, 0), np.float16), np.zeros((90, 0), np.float16))
    assert np.all(d == 0)
    note("acc16 overflow")
    A = np.full((64, 256), 16.0, np.float16)
    assert np.all(_run(A, A) == 0x7C00)
    assert np.all(_run(A, -A) == 0xFC00)
    note("acc16 negative zero")
    # one product per entry, -2^-26: the chunk sum rounds to -0, and
    # +0 + -0 = +0 (the fp32 path writes -0)
    A = np.zeros((64, 64), np.float16)
    A[:, 0] = -(2.0 ** -12)
    Bz = np.full((64, 64), 2.0 ** -14, np.float16)
    assert np.all(_run(A, Bz) == 0)
    assert np.all(run_gemm(A, Bz) == 0x8000)
    import torch
    x = torch.zeros(16, dtype=torch.float16, device="cuda:0")
    p = x.data_ptr()
    assert binding.gemm_nt_f16_acc16(p, p + 32, p, 4, 4, 2, 0) == binding.GEMM_EINVAL
    assert binding.gemm_nt_f16_acc16(p, p, p + 1, 1, 1, 1, 0) == binding.GEMM_EINVAL
    assert binding.gemm_nt_f16_acc16(p, p, p, 0, 3, 3, 0) == binding.GEMM_OK


def test_acc16_deterministic():
    A, B = wl.uniform_inputs(19950, 1024, 1024, 1024)
    note("acc16 determinism")
    d0 = _run(A, B)
    assert np.array_equal(d0, _run(A, B)) and np.array_equal(d0, _run(A, B, repeat=3))
