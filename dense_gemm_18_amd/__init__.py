"""dense_gemm_18_amd -- dense fp16 NT GEMM for AMD MI355X (gfx950).

D[m,n] = sum_k A[m,k] * B[n,k], A stored M x K, B stored N x K, fp16 in and
out, fp32 accumulation, computed by hand-written HIP kernels behind the C ABI
declared in ``include/gemm_nt_f16.h``.  The HIP library is loaded on first
use; a missing library is an error, never a fallback.
"""
from .binding import (GEMM_EINVAL, GEMM_ELAUNCH, GEMM_MAX_K, GEMM_OK, GemmError, gemm_nt,
                      gemm_nt_f16, gemm_nt_f16_strerror, gemm_nt_f16_tile,
                      gemm_nt_f16_tile_coord)

__all__ = ["gemm_nt", "gemm_nt_f16", "gemm_nt_f16_strerror", "gemm_nt_f16_tile",
           "gemm_nt_f16_tile_coord", "GemmError", "GEMM_OK", "GEMM_EINVAL", "GEMM_ELAUNCH",
           "GEMM_MAX_K"]
