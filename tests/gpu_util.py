"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle.

Tolerance for random inputs, evaluated in fp64 on the widened fp16 values:
    |D_gpu - D_ref| <= 2^-10 * |D_ref| + 1e-3 * sqrt(K)
where D_ref is the oracle's fp16 result.  The first term is one fp16
rounding step (half an ulp is 2^-11 relative; the fp32-accumulated sum may
land on the other side of a rounding boundary); the second bounds the fp32
accumulation drift, which grows like sqrt(K) for random signs.  Integer
inputs must match bit for bit: fp32 sums of small integers are exact and
both sides round the same exact value once.
"""
from __future__ import annotations

import math
import sys

import numpy as np

CANARY = 0x7E5A          # a NaN pattern the kernel never writes
GUARD = 256              # guard elements on each side of D (512 B keeps alignment)


def device():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    return torch.device("cuda:0")


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault still shows it."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, misalign_elems: int = 0):
    """Copy fp16 numpy data to the GPU; optionally start it `misalign_elems`
    fp16 elements past a 256-byte boundary (to exercise the general path)."""
    import torch
    dev = device()
    flat = np.ascontiguousarray(x, dtype=np.float16).ravel()
    if misalign_elems == 0:
        return torch.from_numpy(flat.copy()).to(dev).view(x.shape), None
    buf = torch.empty(flat.size + misalign_elems + 8, dtype=torch.float16, device=dev)
    view = buf[misalign_elems: misalign_elems + flat.size]
    view.copy_(torch.from_numpy(flat.copy()).to(dev))
    return view.view(x.shape), buf


def run_gemm(A: np.ndarray, B: np.ndarray, *, a_off: int = 0, b_off: int = 0, d_off: int = 0,
             check_canary: bool = True, repeat: int = 1, acc16: bool = False) -> np.ndarray:
    """D = A B^T on the GPU through the C ABI; returns fp16 bit patterns.

    D lives inside a buffer with GUARD canary elements on both sides; the
    canaries must survive.  `*_off` shift operands by whole fp16 elements.
    acc16: through gemm_nt_f16_acc16 (fp16 running sum) instead."""
    import torch
    from dense_gemm_18_amd import binding

    M, K = A.shape
    N = B.shape[0]
    dev = device()
    dA, _ka = to_dev(A, a_off)
    dB, _kb = to_dev(B, b_off)
    total = M * N + 2 * GUARD + d_off
    dbuf = torch.full((total,), int(np.uint16(CANARY).view(np.int16)), dtype=torch.int16,
                      device=dev)
    dptr = dbuf.data_ptr() + 2 * (GUARD + d_off)
    stream = torch.cuda.current_stream(dev).cuda_stream
    fn = binding.gemm_nt_f16_acc16 if acc16 else binding.gemm_nt_f16
    for _ in range(repeat):
        rc = fn(dA.data_ptr(), dB.data_ptr(), dptr, M, N, K, stream)
        assert rc == binding.GEMM_OK, binding.gemm_nt_f16_strerror(rc)
    torch.cuda.synchronize(dev)
    host = dbuf.cpu().numpy().view(np.uint16)
    if check_canary:
        lo = host[: GUARD + d_off]
        hi = host[GUARD + d_off + M * N:]
        assert np.all(lo == CANARY), "write before D"
        assert np.all(hi == CANARY), "write after D"
    return host[GUARD + d_off: GUARD + d_off + M * N].reshape(M, N).copy()


def run_gemm_ws(A: np.ndarray, B: np.ndarray, workspace=None, ws_bytes=None,
                repeat: int = 1) -> np.ndarray:
    """D = A B^T through the stream-K entry point gemm_nt_f16_ws, with canaries
    around D.  `workspace`: a zero-filled uint8 CUDA tensor (allocated to the
    size the library asks for when None); returns fp16 bit patterns."""
    import torch
    from dense_gemm_18_amd import binding

    M, K = A.shape
    N = B.shape[0]
    dev = device()
    dA, _ = to_dev(A)
    dB, _ = to_dev(B)
    if workspace is None:
        need = binding.gemm_nt_f16_ws_size(M, N, K)
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    if ws_bytes is None:
        ws_bytes = workspace.numel()
    dbuf = torch.full((M * N + 2 * GUARD,), int(np.uint16(CANARY).view(np.int16)),
                      dtype=torch.int16, device=dev)
    dptr = dbuf.data_ptr() + 2 * GUARD
    stream = torch.cuda.current_stream(dev).cuda_stream
    for _ in range(repeat):
        rc = binding.gemm_nt_f16_ws(dA.data_ptr(), dB.data_ptr(), dptr, M, N, K,
                                    workspace.data_ptr(), ws_bytes, stream)
        assert rc == binding.GEMM_OK, binding.gemm_nt_f16_strerror(rc)
    torch.cuda.synchronize(dev)
    host = dbuf.cpu().numpy().view(np.uint16)
    assert np.all(host[:GUARD] == CANARY), "write before D"
    assert np.all(host[GUARD + M * N:] == CANARY), "write after D"
    return host[GUARD: GUARD + M * N].reshape(M, N).copy()


def run_gemm_ex(A: np.ndarray, B: np.ndarray, C=None, bias=None, alpha=1.0, beta=0.0,
                in_place: bool = False) -> np.ndarray:
    """D = alpha A B^T + beta C + bias through gemm_nt_f16_ex, canaries around
    D.  in_place: C is written into D's buffer first and passed as D itself."""
    import torch
    from dense_gemm_18_amd import binding

    M, K = A.shape
    N = B.shape[0]
    dev = device()
    dA, _ = to_dev(A)
    dB, _ = to_dev(B)
    dbuf = torch.full((M * N + 2 * GUARD,), int(np.uint16(CANARY).view(np.int16)),
                      dtype=torch.int16, device=dev)
    dptr = dbuf.data_ptr() + 2 * GUARD
    cptr = 0
    if C is not None:
        c16 = np.ascontiguousarray(C, dtype=np.float16)
        if in_place:
            dbuf[GUARD:GUARD + M * N].copy_(torch.from_numpy(c16.view(np.int16).ravel().copy()))
            cptr = dptr
        else:
            dC, _ = to_dev(c16)
            cptr = dC.data_ptr()
    bptr = 0
    if bias is not None:
        dbias, _ = to_dev(np.ascontiguousarray(bias, dtype=np.float16))
        bptr = dbias.data_ptr()
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = binding.gemm_nt_f16_ex(dA.data_ptr(), dB.data_ptr(), cptr, bptr, dptr, M, N, K,
                                alpha, beta, stream)
    assert rc == binding.GEMM_OK, binding.gemm_nt_f16_strerror(rc)
    torch.cuda.synchronize(dev)
    host = dbuf.cpu().numpy().view(np.uint16)
    assert np.all(host[:GUARD] == CANARY), "write before D"
    assert np.all(host[GUARD + M * N:] == CANARY), "write after D"
    return host[GUARD: GUARD + M * N].reshape(M, N).copy()


def run_gemm_bf16(A: np.ndarray, B: np.ndarray, d_off: int = 0) -> np.ndarray:
    """bfloat16 D = A B^T through gemm_nt_bf16 (uint16 bit patterns in and
    out), canaries around D; D starts `d_off` elements past a 256-byte
    boundary."""
    import torch
    from dense_gemm_18_amd import binding

    M, K = A.shape
    N = B.shape[0]
    dev = device()
    dA = torch.from_numpy(np.ascontiguousarray(A, np.uint16).view(np.int16).copy()).to(dev)
    dB = torch.from_numpy(np.ascontiguousarray(B, np.uint16).view(np.int16).copy()).to(dev)
    g = GUARD + d_off
    dbuf = torch.full((M * N + 2 * GUARD + d_off,), int(np.uint16(CANARY).view(np.int16)),
                      dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = binding.gemm_nt_bf16(dA.data_ptr(), dB.data_ptr(), dbuf.data_ptr() + 2 * g, M, N, K,
                              stream)
    assert rc == binding.GEMM_OK, binding.gemm_nt_f16_strerror(rc)
    torch.cuda.synchronize(dev)
    host = dbuf.cpu().numpy().view(np.uint16)
    assert np.all(host[:g] == CANARY), "write before D"
    assert np.all(host[g + M * N:] == CANARY), "write after D"
    return host[g: g + M * N].reshape(M, N).copy()


def f16val(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def tolerance_report(d_gpu: np.ndarray, d_ref: np.ndarray, K: int, scale: float = 1.0) -> dict:
    """Elementwise tolerance check; returns a summary (ok, counts, worst).
    `scale` multiplies the accumulation term (|alpha| for the fused epilogue,
    which scales the fp32 sum and its drift)."""
    g = f16val(d_gpu)
    r = f16val(d_ref)
    inf_ref = np.isinf(r)
    bound = 2.0 ** -10 * np.abs(r) + 1e-3 * math.sqrt(max(K, 0)) * abs(scale)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - r)
    ok_fin = (~inf_ref) & np.isfinite(g) & (err <= bound)
    ok_inf = inf_ref & (g == r)
    ok = ok_fin | ok_inf
    same = d_gpu == d_ref
    bad = np.flatnonzero(~ok.ravel())
    return {
        "ok": bool(ok.all()),
        "n": int(ok.size),
        "bad": int(bad.size),
        "first_bad": [int(i) for i in bad[:5]],
        "bitwise_equal_frac": float(same.mean()) if same.size else 1.0,
        "max_err": float(np.nanmax(np.where(inf_ref, 0, err))) if err.size else 0.0,
    }


def assert_tolerance(d_gpu, d_ref, K, what="", scale=1.0):
    rep = tolerance_report(d_gpu, d_ref, K, scale)
    note(f"{what}: {rep}")
    assert rep["ok"], f"{what}: {rep['bad']} of {rep['n']} entries outside tolerance {rep}"
    return rep


def assert_bitexact(d_gpu, d_ref, what=""):
    diff = np.flatnonzero(d_gpu.ravel() != d_ref.ravel())
    if diff.size:
        i = diff[0]
        raise AssertionError(f"{what}: {diff.size} entries differ; first flat index {i}: "
                             f"gpu 0x{int(d_gpu.ravel()[i]):04x} ref 0x{int(d_ref.ravel()[i]):04x}")


def run_gemm_fp8(A: np.ndarray, B: np.ndarray, scale: float = 1.0, fa: int = 0, fb: int = 0,
                 a_off: int = 0, b_off: int = 0, d_off: int = 0) -> np.ndarray:
    """D = scale * A B^T through gemm_nt_fp8 (A, B: FP8 bytes, D: fp16 bit
    patterns), canaries around D.  `a_off`, `b_off` start an operand that
    many bytes past a 256-byte boundary; D starts `d_off` fp16 elements past
    one."""
    import torch
    from dense_gemm_18_amd import binding

    M, K = A.shape
    N = B.shape[0]
    dev = device()

    def put(x, off):
        flat = np.ascontiguousarray(x, dtype=np.uint8).ravel()
        buf = torch.zeros(flat.size + off + 16, dtype=torch.uint8, device=dev)
        if flat.size:
            buf[off:off + flat.size].copy_(torch.from_numpy(flat.copy()).to(dev))
        return buf, buf.data_ptr() + off

    _ka, pa = put(A, a_off)
    _kb, pb = put(B, b_off)
    g = GUARD + d_off
    dbuf = torch.full((M * N + 2 * GUARD + d_off,), int(np.uint16(CANARY).view(np.int16)),
                      dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = binding.gemm_nt_fp8(pa, pb, dbuf.data_ptr() + 2 * g, M, N, K, scale, fa, fb, stream)
    assert rc == binding.GEMM_OK, binding.gemm_nt_f16_strerror(rc)
    torch.cuda.synchronize(dev)
    host = dbuf.cpu().numpy().view(np.uint16)
    assert np.all(host[:g] == CANARY), "write before D"
    assert np.all(host[g + M * N:] == CANARY), "write after D"
    return host[g: g + M * N].reshape(M, N).copy()


def run_gemm_fp8_cs(A: np.ndarray, B: np.ndarray, a_scale: float, b_scale: np.ndarray,
                    fa: int = 0, fb: int = 0, d_off: int = 0) -> np.ndarray:
    """D = (a_scale * b_scale[n]) * A B^T through gemm_nt_fp8_cs (A, B: FP8
    bytes, b_scale: N fp32 values copied to the device, D: fp16 bit
    patterns), canaries around D; D starts `d_off` fp16 elements past a
    256-byte boundary."""
    import torch
    from dense_gemm_18_amd import binding

    M, K = A.shape
    N = B.shape[0]
    dev = device()
    dA = torch.from_numpy(np.ascontiguousarray(A, dtype=np.uint8).copy()).to(dev)
    dB = torch.from_numpy(np.ascontiguousarray(B, dtype=np.uint8).copy()).to(dev)
    dS = torch.from_numpy(np.ascontiguousarray(b_scale, dtype=np.float32).copy()).to(dev)
    g = GUARD + d_off
    dbuf = torch.full((M * N + 2 * GUARD + d_off,), int(np.uint16(CANARY).view(np.int16)),
                      dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = binding.gemm_nt_fp8_cs(dA.data_ptr() if A.size else 0, dB.data_ptr() if B.size else 0,
                                dbuf.data_ptr() + 2 * g, M, N, K, a_scale, dS.data_ptr(), fa, fb,
                                stream)
    assert rc == binding.GEMM_OK, binding.gemm_nt_f16_strerror(rc)
    torch.cuda.synchronize(dev)
    host = dbuf.cpu().numpy().view(np.uint16)
    assert np.all(host[:g] == CANARY), "write before D"
    assert np.all(host[g + M * N:] == CANARY), "write after D"
    return host[g: g + M * N].reshape(M, N).copy()
