// gemm_nt_fp8.hip -- C entry points of the FP8 GEMM (gemm_nt_fp8, and
// gemm_nt_fp8_cs with per-channel weight scales) and the launches with B in
// E4M3.  Kernels and helpers: gemm_kernels.h, gemm_fp8.h.
#include "gemm_fp8.h"

namespace {
// Shared by gemm_nt_fp8 (col_scale == nullptr) and gemm_nt_fp8_cs.
int fp8_call(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, float scale,
             const float *col_scale, bool want_cols, int a_format, int b_format,
             hipStream_t stream)
{
    if (!sizes_ok(M, N, K))
        return GEMM_EINVAL;
    if ((a_format != GEMM_FP8_E4M3 && a_format != GEMM_FP8_E5M2) ||
        (b_format != GEMM_FP8_E4M3 && b_format != GEMM_FP8_E5M2))
        return GEMM_EINVAL;
    const uint64_t a_bytes = (uint64_t)M * (uint64_t)K, b_bytes = (uint64_t)N * (uint64_t)K;
    const uint64_t d_bytes = (uint64_t)M * (uint64_t)N * 2u;
    const uint64_t s_bytes = want_cols && M > 0 ? (uint64_t)N * 4u : 0u;
    if ((a_bytes && !A) || (b_bytes && !B) || (d_bytes && !D) || ((uintptr_t)D & 1u))
        return GEMM_EINVAL;
    if (s_bytes && (!col_scale || ((uintptr_t)col_scale & 3u)))
        return GEMM_EINVAL;
    auto overlap = [](const void *p, uint64_t pn, const void *q, uint64_t qn) {
        const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
        return pn && qn && a < b + qn && b < a + pn;
    };
    if (overlap(D, d_bytes, A, a_bytes) || overlap(D, d_bytes, B, b_bytes) ||
        overlap(D, d_bytes, col_scale, s_bytes))
        return GEMM_EINVAL;
    if (M == 0 || N == 0)
        return GEMM_OK;
    if (K == 0) {
        const Epi epi{nullptr, nullptr, scale, 0.0f, col_scale};
        const int64_t count = M * N;
        const int64_t blocks = cdiv(count, 256) < 4096 ? cdiv(count, 256) : 4096;
        hipLaunchKernelGGL(epilogue_only_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (_Float16 *)D, epi, M, N);
    } else {
        switch (1 + a_format + 2 * b_format) {
        case 1: launch_fp8<1>(A, B, D, M, N, K, scale, col_scale, stream); break;
        case 2: launch_fp8<2>(A, B, D, M, N, K, scale, col_scale, stream); break;
        default:
            gemm18_fp8_launch_b5(1 + a_format + 2 * b_format, A, B, D, M, N, K, scale, col_scale,
                                 stream);
        }
    }
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ELAUNCH;
}
} // namespace

extern "C" {
int gemm_nt_fp8(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                float scale, int a_format, int b_format, hipStream_t stream)
{
    return fp8_call(A, B, D, M, N, K, scale, nullptr, false, a_format, b_format, stream);
}

int gemm_nt_fp8_cs(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                   float a_scale, const float *b_scale, int a_format, int b_format,
                   hipStream_t stream)
{
    return fp8_call(A, B, D, M, N, K, a_scale, b_scale, true, a_format, b_format, stream);
}

int gemm_nt_fp8_tile(int64_t M, int64_t N, int64_t K, int aligned16, int *bm, int *bn)
{
    if (!sizes_ok(M, N, K) || !bm || !bn)
        return GEMM_EINVAL;
    // stand-in addresses with the alignment asked about (4-byte otherwise)
    const void *p = (const void *)(uintptr_t)(aligned16 ? 0x1000 : 0x1004);
    const int lb = fp8_load_bytes(p, p, M, N, K);
    tile_dims(fp8_tile(M, N, K, lb), *bm, *bn);
    return GEMM_OK;
}

} // extern "C"
