"""Python binding of the C ABI in ``include/gemm_nt_f16.h``.

Argument marshalling only: every step of the GEMM runs in the HIP kernels of
``libgemm18.so``.  PyTorch supplies device memory and the current stream.
A missing library raises; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

_LIB_PATH = Path(__file__).resolve().parent / "libgemm18.so"
_lib = None

GEMM_OK = 0
GEMM_EINVAL = 1
GEMM_ELAUNCH = 2
GEMM_ESCRATCH = 3
GEMM_MAX_K = 4194303
GEMM_FP8_E4M3 = 0
GEMM_FP8_E5M2 = 1

# Every symbol the header declares.
EXPORTS = ("gemm_nt_f16", "gemm_nt_f16_strerror", "gemm_nt_f16_tile", "gemm_nt_f16_tile_coord",
           "gemm_nt_bf16", "gemm_nt_f16_ex", "gemm_nt_f16_ws", "gemm_nt_f16_ws_size", "gemm_nt_f16_ws_tile",
           "gemm_nt_f16_ws_items", "gemm_nt_fp8", "gemm_nt_fp8_cs", "gemm_nt_fp8_tile",
           "gemm_nt_f16_kernel", "gemm_nt_f16_ws_noalloc", "gemm_nt_f16_acc16",
           "gemm_nt_f16_acc16_kernel")


class GemmError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {gemm_nt_f16_strerror(code)} (code {code})")


def library_path() -> Path:
    return _LIB_PATH


def lib():
    """Load ``libgemm18.so`` (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it first with "
            "`python -c 'import __graft_entry__ as g; g.build()'`")
    # One HIP runtime per process: PyTorch's bundled libamdhip64 must be the
    # one loaded.  The library asks for libamdhip64.so.7, which resolves to
    # an already-loaded runtime of that soname; loaded first, it would pull
    # in the system runtime, and PyTorch (which asks for libamdhip64.so)
    # would then load a second one that finds no device.
    import torch  # noqa: F401
    L = ctypes.CDLL(str(_LIB_PATH))
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.gemm_nt_f16.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    L.gemm_nt_f16.restype = ctypes.c_int
    L.gemm_nt_f16_strerror.argtypes = [ctypes.c_int]
    L.gemm_nt_f16_strerror.restype = ctypes.c_char_p
    ip = ctypes.POINTER(ctypes.c_int)
    lp = ctypes.POINTER(ctypes.c_int64)
    L.gemm_nt_f16_tile.argtypes = [i64, i64, i64, ip, ip, ip, lp]
    L.gemm_nt_f16_tile.restype = ctypes.c_int
    L.gemm_nt_f16_kernel.argtypes = [vp, vp, vp, i64, i64, i64, ip, ip, ip, ip]
    L.gemm_nt_f16_kernel.restype = ctypes.c_int
    L.gemm_nt_f16_tile_coord.argtypes = [i64, i64, i64, lp, lp]
    L.gemm_nt_f16_tile_coord.restype = ctypes.c_int
    L.gemm_nt_f16_acc16.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    L.gemm_nt_f16_acc16.restype = ctypes.c_int
    L.gemm_nt_f16_acc16_kernel.argtypes = [vp, vp, i64, i64, i64, ip, ip, ip]
    L.gemm_nt_f16_acc16_kernel.restype = ctypes.c_int
    L.gemm_nt_bf16.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    L.gemm_nt_bf16.restype = ctypes.c_int
    L.gemm_nt_f16_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_float,
                                 ctypes.c_float, vp]
    L.gemm_nt_f16_ex.restype = ctypes.c_int
    L.gemm_nt_f16_ws.argtypes = [vp, vp, vp, i64, i64, i64, vp, i64, vp]
    L.gemm_nt_f16_ws.restype = ctypes.c_int
    L.gemm_nt_f16_ws_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    L.gemm_nt_f16_ws_noalloc.restype = ctypes.c_int
    L.gemm_nt_f16_ws_size.argtypes = [i64, i64, i64]
    L.gemm_nt_f16_ws_size.restype = i64
    L.gemm_nt_f16_ws_tile.argtypes = [i64, i64, i64, ip, ip, lp, lp]
    L.gemm_nt_f16_ws_tile.restype = ctypes.c_int
    L.gemm_nt_f16_ws_items.argtypes = [i64, i64, i64, i64, lp, i64, lp]
    L.gemm_nt_f16_ws_items.restype = ctypes.c_int
    L.gemm_nt_fp8.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                              ctypes.c_int, vp]
    L.gemm_nt_fp8.restype = ctypes.c_int
    L.gemm_nt_fp8_cs.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_float, vp, ctypes.c_int,
                                 ctypes.c_int, vp]
    L.gemm_nt_fp8_cs.restype = ctypes.c_int
    L.gemm_nt_fp8_tile.argtypes = [i64, i64, i64, ctypes.c_int, ip, ip]
    L.gemm_nt_fp8_tile.restype = ctypes.c_int
    _lib = L
    return L


# ---- the C entry points, same names ---------------------------------------

def gemm_nt_f16(A: int, B: int, D: int, M: int, N: int, K: int, stream: int = 0) -> int:
    """Raw call: device addresses as integers; returns the C return code."""
    return lib().gemm_nt_f16(A or None, B or None, D or None, M, N, K, stream or None)


def gemm_nt_f16_strerror(code: int) -> str:
    return lib().gemm_nt_f16_strerror(code).decode()


def gemm_nt_f16_tile(M: int, N: int, K: int):
    """(BM, BN, BK, workgroups) the library uses for an M x N x K problem."""
    bm, bn, bk = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    wg = ctypes.c_int64()
    rc = lib().gemm_nt_f16_tile(M, N, K, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(bk),
                                ctypes.byref(wg))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_nt_f16_tile")
    return bm.value, bn.value, bk.value, wg.value


def gemm_nt_f16_kernel(A: int, B: int, D: int, M: int, N: int, K: int):
    """(BM, BN, load_bytes, store_mode) of the kernel a gemm_nt_f16 call with
    these device addresses and sizes takes (host-only, nothing is read)."""
    bm, bn, lb, st = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rc = lib().gemm_nt_f16_kernel(A or None, B or None, D or None, M, N, K, ctypes.byref(bm),
                                  ctypes.byref(bn), ctypes.byref(lb), ctypes.byref(st))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_nt_f16_kernel")
    return bm.value, bn.value, lb.value, st.value


def gemm_nt_f16_acc16(A: int, B: int, D: int, M: int, N: int, K: int, stream: int = 0) -> int:
    """Raw call of the fp16-accumulating product; returns the C return code."""
    return lib().gemm_nt_f16_acc16(A or None, B or None, D or None, M, N, K, stream or None)


def gemm_nt_f16_acc16_kernel(A: int, B: int, M: int, N: int, K: int):
    """(BM, BN, load_bytes) of the kernel a gemm_nt_f16_acc16 call with these
    device addresses and sizes takes (host-only, nothing is read)."""
    bm, bn, lb = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rc = lib().gemm_nt_f16_acc16_kernel(A or None, B or None, M, N, K, ctypes.byref(bm),
                                        ctypes.byref(bn), ctypes.byref(lb))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_nt_f16_acc16_kernel")
    return bm.value, bn.value, lb.value


def gemm_nt_f16_tile_coord(wg: int, tiles_m: int, tiles_n: int):
    """(tile_m, tile_n) computed by workgroup ``wg``."""
    tm, tn = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().gemm_nt_f16_tile_coord(wg, tiles_m, tiles_n, ctypes.byref(tm), ctypes.byref(tn))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_nt_f16_tile_coord")
    return tm.value, tn.value


def gemm_nt_bf16(A: int, B: int, D: int, M: int, N: int, K: int, stream: int = 0) -> int:
    """Raw call of the bfloat16 form; returns the C return code."""
    return lib().gemm_nt_bf16(A or None, B or None, D or None, M, N, K, stream or None)


def gemm_nt_f16_ex(A: int, B: int, C: int, bias: int, D: int, M: int, N: int, K: int,
                   alpha: float = 1.0, beta: float = 0.0, stream: int = 0) -> int:
    """Raw call of the fused-epilogue form (C, bias: 0 for none)."""
    return lib().gemm_nt_f16_ex(A or None, B or None, C or None, bias or None, D or None,
                                M, N, K, alpha, beta, stream or None)


def gemm_nt_f16_ws(A: int, B: int, D: int, M: int, N: int, K: int, workspace: int,
                   ws_bytes: int, stream: int = 0) -> int:
    """Raw call of the stream-K form; returns the C return code."""
    return lib().gemm_nt_f16_ws(A or None, B or None, D or None, M, N, K, workspace or None,
                                ws_bytes, stream or None)


def gemm_nt_f16_ws_noalloc(A: int, B: int, D: int, M: int, N: int, K: int,
                           stream: int = 0) -> int:
    """Raw call of the stream-K form on the library's static scratch (no
    allocation); returns the C return code."""
    return lib().gemm_nt_f16_ws_noalloc(A or None, B or None, D or None, M, N, K, stream or None)


def gemm_nt_f16_ws_size(M: int, N: int, K: int) -> int:
    return lib().gemm_nt_f16_ws_size(M, N, K)


def gemm_nt_f16_ws_tile(M: int, N: int, K: int):
    """(BM, BN, workgroups, stream-K tiles) of the stream-K form's plan."""
    bm, bn = ctypes.c_int(), ctypes.c_int()
    wg, skt = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().gemm_nt_f16_ws_tile(M, N, K, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(wg),
                                   ctypes.byref(skt))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_nt_f16_ws_tile")
    return bm.value, bn.value, wg.value, skt.value


def gemm_nt_f16_ws_items(M: int, N: int, K: int, wg: int):
    """Work items (tile, s0, s1, w_first, w_last) of workgroup ``wg``."""
    count = ctypes.c_int64()
    rc = lib().gemm_nt_f16_ws_items(M, N, K, wg, None, 0, ctypes.byref(count))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_nt_f16_ws_items")
    buf = (ctypes.c_int64 * (5 * max(count.value, 1)))()
    rc = lib().gemm_nt_f16_ws_items(M, N, K, wg, buf, count.value, ctypes.byref(count))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_nt_f16_ws_items")
    return [tuple(buf[5 * i:5 * i + 5]) for i in range(count.value)]


def gemm_nt_fp8(A: int, B: int, D: int, M: int, N: int, K: int, scale: float = 1.0,
                a_format: int = GEMM_FP8_E4M3, b_format: int = GEMM_FP8_E4M3,
                stream: int = 0) -> int:
    """Raw call of the FP8 form (A, B: FP8 bytes, D: fp16); returns the C
    return code."""
    return lib().gemm_nt_fp8(A or None, B or None, D or None, M, N, K, scale, a_format,
                             b_format, stream or None)


def gemm_nt_fp8_cs(A: int, B: int, D: int, M: int, N: int, K: int, a_scale: float,
                   b_scale: int, a_format: int = GEMM_FP8_E4M3, b_format: int = GEMM_FP8_E4M3,
                   stream: int = 0) -> int:
    """Raw call of the FP8 form with per-channel weight scales (b_scale: device
    address of N fp32 values, one per row of B); returns the C return code."""
    return lib().gemm_nt_fp8_cs(A or None, B or None, D or None, M, N, K, a_scale,
                                b_scale or None, a_format, b_format, stream or None)


def gemm_nt_fp8_tile(M: int, N: int, K: int, aligned16: bool = True):
    """(BM, BN) of the FP8 form's tile; (0, 0) for the plain kernel."""
    bm, bn = ctypes.c_int(), ctypes.c_int()
    rc = lib().gemm_nt_fp8_tile(M, N, K, int(bool(aligned16)), ctypes.byref(bm), ctypes.byref(bn))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_nt_fp8_tile")
    return bm.value, bn.value


# ---- tensor-level convenience ----------------------------------------------

def gemm_nt(A, B, out=None, stream=None, scale: float = 1.0, b_scale=None):
    """D = A @ B.T for CUDA (HIP) tensors A [M, K] and B [N, K].

    float16 A and B call gemm_nt_f16 (D float16), bfloat16 call gemm_nt_bf16
    (D bfloat16); float8_e4m3fn / float8_e5m2 operands (the two may differ)
    call gemm_nt_fp8 with ``scale`` (D float16), or, given ``b_scale`` (a
    contiguous float32 tensor of N per-row scales of B on the same device),
    gemm_nt_fp8_cs with a_scale = ``scale``.  ``out`` (optional) is a
    contiguous [M, N] tensor of D's dtype on the same device.  The call is
    enqueued on ``stream`` (default: A's device's current stream; a stream
    given must belong to A's device), with A's device made current for it.
    """
    import torch

    fp8 = {torch.float8_e4m3fn: GEMM_FP8_E4M3, torch.float8_e5m2: GEMM_FP8_E5M2}
    if A.dtype in fp8 and B.dtype in fp8:
        out_dtype = torch.float16
    elif A.dtype == B.dtype and A.dtype in (torch.float16, torch.bfloat16):
        out_dtype = A.dtype
    else:
        raise TypeError(f"unsupported operand dtypes {A.dtype} and {B.dtype}: both float16, "
                        "both bfloat16, or float8_e4m3fn / float8_e5m2")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError(f"shapes {tuple(A.shape)} and {tuple(B.shape)} are not [M,K] and [N,K]")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("A and B must be on the same GPU")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous row-major")
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    elif (out.dtype != out_dtype or tuple(out.shape) != (M, N) or not out.is_contiguous()
          or out.device != A.device):
        raise ValueError(f"out must be a contiguous {out_dtype} [M, N] tensor on A's device")
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    pa, pb, pd = A.data_ptr(), B.data_ptr(), out.data_ptr()
    if b_scale is not None:
        if A.dtype not in fp8:
            raise TypeError("b_scale applies to FP8 operands only")
        if (b_scale.dtype != torch.float32 or b_scale.numel() != N or not b_scale.is_contiguous()
                or b_scale.device != A.device):
            raise ValueError("b_scale must be a contiguous float32 tensor of N values on A's device")
    # the library launches on the current device: make it the operands' one
    with torch.cuda.device(A.device):
        if A.dtype in fp8 and b_scale is not None:
            name = "gemm_nt_fp8_cs"
            rc = gemm_nt_fp8_cs(pa, pb, pd, M, N, K, scale, b_scale.data_ptr(), fp8[A.dtype],
                                fp8[B.dtype], s.cuda_stream)
        elif A.dtype in fp8:
            name = "gemm_nt_fp8"
            rc = gemm_nt_fp8(pa, pb, pd, M, N, K, scale, fp8[A.dtype], fp8[B.dtype],
                             s.cuda_stream)
        elif A.dtype == torch.bfloat16:
            name = "gemm_nt_bf16"
            rc = gemm_nt_bf16(pa, pb, pd, M, N, K, s.cuda_stream)
        else:
            name = "gemm_nt_f16"
            rc = gemm_nt_f16(pa, pb, pd, M, N, K, s.cuda_stream)
    if rc != GEMM_OK:
        raise GemmError(rc, name)
    return out
