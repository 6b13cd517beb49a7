// gemm_nt_f16_ex.hip -- C entry point of the fp16 GEMM with the fused
// epilogue (gemm_nt_f16_ex).
// Kernels, tile choice and launch helpers are in gemm_kernels.h.
#include "gemm_kernels.h"

extern "C" {
int gemm_nt_f16_ex(const void *A, const void *B, const void *C, const void *bias, void *D,
                   int64_t M, int64_t N, int64_t K, float alpha, float beta, hipStream_t stream)
{
    int rc = validate(A, B, D, M, N, K);
    if (rc != GEMM_OK)
        return rc;
    const uint64_t d_bytes = (uint64_t)M * (uint64_t)N * 2u;
    auto overlaps_d = [&](const void *p, uint64_t bytes) {
        const uintptr_t a = (uintptr_t)p, d = (uintptr_t)D;
        return bytes && d_bytes && a < d + d_bytes && d < a + bytes;
    };
    if (beta != 0.0f) {
        if ((d_bytes && !C) || ((uintptr_t)C & 1u) || (C != D && overlaps_d(C, d_bytes)))
            return GEMM_EINVAL;
    } else {
        C = nullptr;                      // not read
    }
    if (bias && (((uintptr_t)bias & 1u) || overlaps_d(bias, (uint64_t)N * 2u)))
        return GEMM_EINVAL;
    if (M == 0 || N == 0)
        return GEMM_OK;
    if (alpha == 1.0f && !C && !bias)
        return gemm_nt_f16(A, B, D, M, N, K, stream);
    const Epi epi{(const _Float16 *)C, (const _Float16 *)bias, alpha, beta};
    if (K == 0) {
        const int64_t count = M * N;
        const int64_t blocks = cdiv(count, 256) < 4096 ? cdiv(count, 256) : 4096;
        hipLaunchKernelGGL(epilogue_only_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (_Float16 *)D, epi, M, N);
    } else {
        launch_plain<true>(choose_tile(M, N, K), A, B, D, (int)M, (int)N, (int)K, stream,
                          epi);
    }
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ELAUNCH;
}

} // extern "C"
