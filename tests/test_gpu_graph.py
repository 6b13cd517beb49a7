"""The C entry points captured in a HIP graph and replayed.

The plain, fp16-accumulating, FP8 and fused-epilogue entry points launch
kernels only (K = 0 writes D with a fill kernel, never hipMemsetAsync), and
the stream-K form keeps its state in the workspace (an epoch per call, reset
by its last workgroup), so all of them can be captured.  Each graph is
replayed several times with eager work and synchronisations in between, D
is cleared before every replay, and every replay must equal the eager result
bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

from dense_gemm_18_amd import binding
from dense_gemm_18_amd import workloads as wl
from tests.gpu_util import note

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _check_graph(call, out):
    """call(stream) enqueues the work writing `out`; eager once, then capture
    and replay, comparing every replay with the eager bits."""
    import torch
    s = torch.cuda.current_stream().cuda_stream
    out.fill_(7)
    assert call(s) == binding.GEMM_OK
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            rc = call(torch.cuda.current_stream().cuda_stream)
    assert rc == binding.GEMM_OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        out.fill_(7)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r} differs"
    del g


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 1024), (2900, 4100, 97), (64, 3000, 448),
                                   (2100, 2200, 1032)])
def test_graph_plain(M, N, K):
    import torch
    A, B = wl.uniform_inputs(21000 + K, M, N, K)
    dA, dB = _dev(A), _dev(B)
    dD = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    note(f"graph gemm_nt_f16 {M}x{N}x{K}")
    _check_graph(lambda s: binding.gemm_nt_f16(dA.data_ptr(), dB.data_ptr(), dD.data_ptr(),
                                               M, N, K, s), dD)


def test_graph_k_zero():
    import torch
    dD = torch.empty((300, 200), dtype=torch.float16, device="cuda:0")
    x = torch.zeros(16, dtype=torch.float16, device="cuda:0")
    note("graph gemm_nt_f16 K=0")
    _check_graph(lambda s: binding.gemm_nt_f16(x.data_ptr(), x.data_ptr(), dD.data_ptr(),
                                               300, 200, 0, s), dD)


def test_graph_acc16():
    import torch
    M, N, K = 2900, 4100, 512
    A, B = wl.coarse_uniform(21500, M, N, K)
    dA, dB = _dev(A), _dev(B)
    dD = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    note(f"graph gemm_nt_f16_acc16 {M}x{N}x{K}")
    _check_graph(lambda s: binding.gemm_nt_f16_acc16(dA.data_ptr(), dB.data_ptr(), dD.data_ptr(),
                                                     M, N, K, s), dD)


def test_graph_fp8_and_epilogue():
    import torch
    M, N, K = 1000, 1100, 1024
    A, B, scale = wl.fp8_normal(21600, M, N, K)
    dA, dB = _dev(A), _dev(B)
    dD = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    note(f"graph gemm_nt_fp8 {M}x{N}x{K}")
    e4 = binding.GEMM_FP8_E4M3
    _check_graph(lambda s: binding.gemm_nt_fp8(dA.data_ptr(), dB.data_ptr(), dD.data_ptr(), M, N,
                                               K, scale, e4, e4, s), dD)
    A2, B2 = wl.uniform_inputs(21700, M, N, K)
    dA2, dB2 = _dev(A2), _dev(B2)
    C = _dev(np.random.default_rng(21701).uniform(-1, 1, (M, N)).astype(np.float16))
    bias = _dev(np.random.default_rng(21702).uniform(-1, 1, N).astype(np.float16))
    note(f"graph gemm_nt_f16_ex {M}x{N}x{K}")
    _check_graph(lambda s: binding.gemm_nt_f16_ex(dA2.data_ptr(), dB2.data_ptr(), C.data_ptr(),
                                                  bias.data_ptr(), dD.data_ptr(), M, N, K, 0.5,
                                                  -1.0, s), dD)


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 12288), (64, 2048, 8192)])
def test_graph_stream_k(M, N, K):
    # the workspace's epochs carry over from call to call and from replay to
    # replay; its header must show no timeout afterwards (128 x 128 and
    # skinny 64 x 32 plans)
    import torch
    A, B = wl.uniform_inputs(21800, M, N, K)
    dA, dB = _dev(A), _dev(B)
    dD = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    need = binding.gemm_nt_f16_ws_size(M, N, K)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    note(f"graph gemm_nt_f16_ws {M}x{N}x{K}")
    _check_graph(lambda s: binding.gemm_nt_f16_ws(dA.data_ptr(), dB.data_ptr(), dD.data_ptr(), M,
                                                  N, K, ws.data_ptr(), need, s), dD)
    hdr = ws[:256].view(torch.int32).cpu().numpy()
    assert hdr[2] == 0, "an owner gave up waiting"
    assert hdr[1] == 0, "done counter not reset"
