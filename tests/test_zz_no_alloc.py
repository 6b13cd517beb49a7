"""GPU check of gemm_nt_f16_ws_noalloc, the stream-K entry point that
allocates nothing (its workspace is the library's static device array),
against gemm_nt_f16_ws with a caller workspace: the same plan and kernels,
so the results must be identical bit for bit.  Two calls in a row share the
static array, the second with a smaller problem; integer inputs are also
compared with the oracle (exact sums: bit-exact).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from dense_gemm_18_amd import binding
from dense_gemm_18_amd import workloads as wl
from tests.gpu_util import CANARY, GUARD, assert_bitexact, note, run_gemm_ws, to_dev

pytestmark = pytest.mark.gpu


def _run_noalloc(A, B):
    import torch
    M, K = A.shape
    N = B.shape[0]
    dev = torch.device("cuda:0")
    dA, _ = to_dev(A)
    dB, _ = to_dev(B)
    dbuf = torch.full((M * N + 2 * GUARD,), int(np.uint16(CANARY).view(np.int16)),
                      dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = binding.gemm_nt_f16_ws_noalloc(dA.data_ptr(), dB.data_ptr(), dbuf.data_ptr() + 2 * GUARD,
                                        M, N, K, stream)
    assert rc == binding.GEMM_OK, binding.gemm_nt_f16_strerror(rc)
    torch.cuda.synchronize(dev)
    host = dbuf.cpu().numpy().view(np.uint16)
    assert np.all(host[:GUARD] == CANARY), "write before D"
    assert np.all(host[GUARD + M * N:] == CANARY), "write after D"
    return host[GUARD: GUARD + M * N].reshape(M, N).copy()


# Two stream-K shapes (the second smaller), then one the plain kernel serves.
SHAPES = [(1024, 1024, 16384), (512, 640, 12288)]


def test_noalloc_matches_workspace_form_two_calls():
    for i, (M, N, K) in enumerate(SHAPES):
        assert binding.gemm_nt_f16_ws_tile(M, N, K)[3] > 0, "shape must take stream-K"
        A, B = wl.uniform_inputs(17000 + i, M, N, K)
        note(f"noalloc random call {i}: {M}x{N}x{K}")
        got = _run_noalloc(A, B)
        want = run_gemm_ws(A, B)
        assert_bitexact(got, want, f"noalloc vs workspace {M}x{N}x{K}")


def test_noalloc_integer_against_oracle_two_calls():
    for i, (M, N, K) in enumerate(SHAPES):
        A, B = wl.integer_free(17100 + i, M, N, K)
        note(f"noalloc integer call {i}: {M}x{N}x{K}")
        got = _run_noalloc(A, B)
        assert_bitexact(got, oracle.gemm_nt_f16(A, B), f"noalloc integer {M}x{N}x{K}")
        assert_bitexact(got, run_gemm_ws(A, B), f"noalloc vs workspace integer {M}x{N}x{K}")


def test_noalloc_skinny_plans_two_calls():
    # skinny stream-K plans on 64 x 64 and 64 x 32 tiles (smaller slots in
    # the same static array), the second call smaller than the first
    for i, (M, N, K) in enumerate([(8192, 64, 8192), (64, 2048, 4096)]):
        assert binding.gemm_nt_f16_ws_tile(M, N, K)[3] > 0, "shape must take stream-K"
        A, B = wl.integer_free(17300 + i, M, N, K)
        note(f"noalloc skinny call {i}: {M}x{N}x{K}")
        got = _run_noalloc(A, B)
        assert_bitexact(got, run_gemm_ws(A, B), f"noalloc vs workspace {M}x{N}x{K}")
        assert_bitexact(got, oracle.gemm_nt_f16(A, B), f"noalloc skinny integer {M}x{N}x{K}")


def test_noalloc_plain_shape_falls_through():
    M, N, K = 300, 200, 96           # not a stream-K plan: runs as gemm_nt_f16
    assert binding.gemm_nt_f16_ws_tile(M, N, K)[3] == 0
    A, B = wl.integer_free(17200, M, N, K)
    note(f"noalloc plain {M}x{N}x{K}")
    assert_bitexact(_run_noalloc(A, B), oracle.gemm_nt_f16(A, B), "noalloc plain shape")
