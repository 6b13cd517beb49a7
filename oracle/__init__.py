"""CPU oracle for the dense fp16 NT GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path (the HIP
library and its Python binding) never imports, calls or loads it, and the
oracle shares no code with that path.

The arithmetic lives in ``gemm_oracle.c`` (plain C, built with gcc, fp64):
``D[m,n] = sum_k A[m,k] * B[n,k]`` with A stored M x K and B stored N x K,
as defined on page "构建 Tiled GEMM" ("Building a Tiled GEMM", mlc.ai
modern-gpu-programming-for-mlsys, chapter gemm_basics), section "GEMM".
Each fp16 input is widened to fp64 exactly, the sum runs over ascending k in
fp64 from +0.0 and is rounded once to fp16 (round to nearest, ties to even).
This module only marshals numpy arrays of raw fp16 bit patterns (uint16).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "gemm_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra"]
_lib = None


def build(force: bool = True) -> Path:
    """Compile ``gemm_oracle.c`` into ``liboracle.so`` with gcc."""
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(f".so.tmp{os.getpid()}")
        subprocess.check_call(["gcc", *_CFLAGS, str(_SRC), "-o", str(tmp), "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        build(force=True)
    lib = ctypes.CDLL(str(_LIB_PATH))
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_f16_decode.argtypes = [p, p, i64]
    lib.oracle_f16_decode.restype = None
    lib.oracle_f16_encode.argtypes = [p, p, i64]
    lib.oracle_f16_encode.restype = None
    lib.oracle_gemm_nt_f16.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int]
    lib.oracle_gemm_nt_f16.restype = ctypes.c_int
    lib.oracle_gemm_nt_f16_entries.argtypes = [p, p, i64, i64, i64, p, p, i64, p, ctypes.c_int]
    lib.oracle_gemm_nt_f16_entries.restype = ctypes.c_int
    lib.oracle_gemm_nt_f16_ex.argtypes = [p, p, p, p, p, i64, i64, i64, ctypes.c_float,
                                          ctypes.c_float, ctypes.c_int]
    lib.oracle_gemm_nt_f16_ex.restype = ctypes.c_int
    lib.oracle_gemm_nt_f16_acc16.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int]
    lib.oracle_gemm_nt_f16_acc16.restype = ctypes.c_int
    lib.oracle_gemm_nt_f16_acc16_entries.argtypes = [p, p, i64, i64, i64, p, p, i64, p,
                                                     ctypes.c_int]
    lib.oracle_gemm_nt_f16_acc16_entries.restype = ctypes.c_int
    lib.oracle_bf16_decode.argtypes = [p, p, i64]
    lib.oracle_bf16_decode.restype = None
    lib.oracle_bf16_encode.argtypes = [p, p, i64]
    lib.oracle_bf16_encode.restype = None
    lib.oracle_gemm_nt_bf16.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int]
    lib.oracle_gemm_nt_bf16.restype = ctypes.c_int
    lib.oracle_gemm_nt_bf16_entries.argtypes = [p, p, i64, i64, i64, p, p, i64, p, ctypes.c_int]
    lib.oracle_gemm_nt_bf16_entries.restype = ctypes.c_int
    lib.oracle_fp8_decode.argtypes = [p, p, i64, ctypes.c_int]
    lib.oracle_fp8_decode.restype = None
    lib.oracle_gemm_nt_fp8.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_float, ctypes.c_int]
    lib.oracle_gemm_nt_fp8.restype = ctypes.c_int
    lib.oracle_gemm_nt_fp8_cs.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_float, p, ctypes.c_int]
    lib.oracle_gemm_nt_fp8_cs.restype = ctypes.c_int
    _lib = lib
    return lib


def _bits(x: np.ndarray) -> np.ndarray:
    """Return a C-contiguous uint16 view of fp16 data (float16 or uint16 in)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16)
    if x.dtype != np.uint16:
        raise TypeError(f"expected float16 or uint16 bit patterns, got {x.dtype}")
    return x


def _ptr(x: np.ndarray) -> int:
    return x.ctypes.data


def decode(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> exact fp64 values (binary16 definition)."""
    b = _bits(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_f16_decode(_ptr(b), _ptr(out), b.size)
    return out


def encode(values: np.ndarray) -> np.ndarray:
    """fp64 values -> fp16 bit patterns, round to nearest, ties to even."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_f16_encode(_ptr(v), _ptr(out), v.size)
    return out


def gemm_nt_f16(A: np.ndarray, B: np.ndarray, threads: int = 0) -> np.ndarray:
    """Full D = A * B^T as fp16 bit patterns (uint16, shape M x N)."""
    a, b = _bits(A), _bits(B)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {a.shape} and {b.shape} are not M x K and N x K")
    M, K = a.shape
    N = b.shape[0]
    d = np.empty((M, N), dtype=np.uint16)
    _load().oracle_gemm_nt_f16(_ptr(a), _ptr(b), _ptr(d), M, N, K, int(threads))
    return d


def gemm_nt_f16_entries(A: np.ndarray, B: np.ndarray, rows, cols,
                        threads: int = 0) -> np.ndarray:
    """Entries D[rows[i], cols[i]] as fp16 bit patterns (uint16, 1-D)."""
    a, b = _bits(A), _bits(B)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {a.shape} and {b.shape} are not M x K and N x K")
    r = np.ascontiguousarray(rows, dtype=np.int64).ravel()
    c = np.ascontiguousarray(cols, dtype=np.int64).ravel()
    if r.shape != c.shape:
        raise ValueError("rows and cols differ in length")
    M, K = a.shape
    N = b.shape[0]
    if r.size and (r.min() < 0 or r.max() >= M or c.min() < 0 or c.max() >= N):
        raise IndexError("entry index outside D")
    out = np.empty(r.shape, dtype=np.uint16)
    _load().oracle_gemm_nt_f16_entries(_ptr(a), _ptr(b), M, N, K, _ptr(r), _ptr(c),
                                       r.size, _ptr(out), int(threads))
    return out


def gemm_nt_f16_acc16(A: np.ndarray, B: np.ndarray, threads: int = 0) -> np.ndarray:
    """D = A * B^T with an fp16 running sum (page "如何用 Croqtile 一步步优化矩阵
    乘法内核", the f16 accumulator of its kernels): chunks of 64 consecutive k,
    aligned to K's end; each chunk's sum is rounded to fp16 and added to the
    fp16 sum with an fp16 addition.  fp16 bit patterns (uint16, M x N)."""
    a, b = _bits(A), _bits(B)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {a.shape} and {b.shape} are not M x K and N x K")
    M, K = a.shape
    N = b.shape[0]
    d = np.empty((M, N), dtype=np.uint16)
    _load().oracle_gemm_nt_f16_acc16(_ptr(a), _ptr(b), _ptr(d), M, N, K, int(threads))
    return d


def gemm_nt_f16_acc16_entries(A: np.ndarray, B: np.ndarray, rows, cols,
                              threads: int = 0) -> np.ndarray:
    """Entries D[rows[i], cols[i]] of the fp16-accumulated product."""
    a, b = _bits(A), _bits(B)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {a.shape} and {b.shape} are not M x K and N x K")
    r = np.ascontiguousarray(rows, dtype=np.int64).ravel()
    c = np.ascontiguousarray(cols, dtype=np.int64).ravel()
    if r.shape != c.shape:
        raise ValueError("rows and cols differ in length")
    M, K = a.shape
    N = b.shape[0]
    if r.size and (r.min() < 0 or r.max() >= M or c.min() < 0 or c.max() >= N):
        raise IndexError("entry index outside D")
    out = np.empty(r.shape, dtype=np.uint16)
    _load().oracle_gemm_nt_f16_acc16_entries(_ptr(a), _ptr(b), M, N, K, _ptr(r), _ptr(c),
                                             r.size, _ptr(out), int(threads))
    return out


def gemm_nt_f16_ex(A: np.ndarray, B: np.ndarray, C=None, bias=None, alpha: float = 1.0,
                   beta: float = 0.0, threads: int = 0) -> np.ndarray:
    """D = alpha * A * B^T + beta * C + bias (bias per column) as fp16 bit
    patterns.  alpha and beta are taken as fp32 values; C is not read when
    beta == 0."""
    a, b = _bits(A), _bits(B)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {a.shape} and {b.shape} are not M x K and N x K")
    M, K = a.shape
    N = b.shape[0]
    alpha32, beta32 = float(np.float32(alpha)), float(np.float32(beta))
    c = None
    if beta32 != 0.0:
        if C is None:
            raise ValueError("beta != 0 needs C")
        c = _bits(C)
        if c.shape != (M, N):
            raise ValueError(f"C has shape {c.shape}, expected {(M, N)}")
    bb = None
    if bias is not None:
        bb = _bits(bias).ravel()
        if bb.size != N:
            raise ValueError(f"bias has {bb.size} entries, expected {N}")
    d = np.empty((M, N), dtype=np.uint16)
    _load().oracle_gemm_nt_f16_ex(_ptr(a), _ptr(b), _ptr(c) if c is not None else None,
                                  _ptr(bb) if bb is not None else None, _ptr(d), M, N, K,
                                  alpha32, beta32, int(threads))
    return d


def _u16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {x.dtype}")
    return x


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact fp64 values."""
    b = _u16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_bf16_decode(_ptr(b), _ptr(out), b.size)
    return out


def bf16_encode(values: np.ndarray) -> np.ndarray:
    """fp64 values -> bfloat16 bit patterns, round to nearest, ties to even."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_bf16_encode(_ptr(v), _ptr(out), v.size)
    return out


def gemm_nt_bf16(A: np.ndarray, B: np.ndarray, threads: int = 0) -> np.ndarray:
    """Full D = A * B^T on bfloat16 bit patterns (uint16 in, uint16 out)."""
    a, b = _u16(A), _u16(B)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {a.shape} and {b.shape} are not M x K and N x K")
    M, K = a.shape
    N = b.shape[0]
    d = np.empty((M, N), dtype=np.uint16)
    _load().oracle_gemm_nt_bf16(_ptr(a), _ptr(b), _ptr(d), M, N, K, int(threads))
    return d


def gemm_nt_bf16_entries(A: np.ndarray, B: np.ndarray, rows, cols, threads: int = 0):
    """Entries D[rows[i], cols[i]] of the bfloat16 product (uint16, 1-D)."""
    a, b = _u16(A), _u16(B)
    r = np.ascontiguousarray(rows, dtype=np.int64).ravel()
    c = np.ascontiguousarray(cols, dtype=np.int64).ravel()
    M, K = a.shape
    N = b.shape[0]
    if r.size and (r.min() < 0 or r.max() >= M or c.min() < 0 or c.max() >= N):
        raise IndexError("entry index outside D")
    out = np.empty(r.shape, dtype=np.uint16)
    _load().oracle_gemm_nt_bf16_entries(_ptr(a), _ptr(b), M, N, K, _ptr(r), _ptr(c), r.size,
                                        _ptr(out), int(threads))
    return out


def fp8_decode(bits: np.ndarray, e5m2: bool = False) -> np.ndarray:
    """FP8 bit patterns (uint8, OCP E4M3 or E5M2) -> exact fp64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint8)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_fp8_decode(_ptr(b), _ptr(out), b.size, int(bool(e5m2)))
    return out


def gemm_nt_fp8(A: np.ndarray, B: np.ndarray, scale: float = 1.0, a_e5m2: bool = False,
                b_e5m2: bool = False, threads: int = 0) -> np.ndarray:
    """D = scale * A * B^T, A and B FP8 bit patterns (uint8), D fp16 bits."""
    a = np.ascontiguousarray(A, dtype=np.uint8)
    b = np.ascontiguousarray(B, dtype=np.uint8)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {a.shape} and {b.shape} are not M x K and N x K")
    M, K = a.shape
    N = b.shape[0]
    d = np.empty((M, N), dtype=np.uint16)
    _load().oracle_gemm_nt_fp8(_ptr(a), _ptr(b), _ptr(d), M, N, K, int(bool(a_e5m2)),
                               int(bool(b_e5m2)), float(np.float32(scale)), int(threads))
    return d


def gemm_nt_fp8_cs(A: np.ndarray, B: np.ndarray, a_scale: float, b_scale: np.ndarray,
                   a_e5m2: bool = False, b_e5m2: bool = False, threads: int = 0) -> np.ndarray:
    """D[m, n] = (a_scale * b_scale[n]) * (A B^T)[m, n], the per-column scale
    formed in fp32; A and B FP8 bit patterns (uint8), b_scale N fp32 values
    (one per row of B), D fp16 bits."""
    a = np.ascontiguousarray(A, dtype=np.uint8)
    b = np.ascontiguousarray(B, dtype=np.uint8)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shapes {a.shape} and {b.shape} are not M x K and N x K")
    M, K = a.shape
    N = b.shape[0]
    s = np.ascontiguousarray(b_scale, dtype=np.float32).ravel()
    if s.size != N:
        raise ValueError(f"b_scale has {s.size} values, B has {N} rows")
    d = np.empty((M, N), dtype=np.uint16)
    _load().oracle_gemm_nt_fp8_cs(_ptr(a), _ptr(b), _ptr(d), M, N, K, int(bool(a_e5m2)),
                                  int(bool(b_e5m2)), float(np.float32(a_scale)), _ptr(s),
                                  int(threads))
    return d


def threads_available() -> int:
    """Host threads OpenMP would use by default (the CPU-baseline core count)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
