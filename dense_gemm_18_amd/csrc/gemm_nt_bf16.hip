// gemm_nt_bf16.hip -- C entry point of the bfloat16 GEMM (gemm_nt_bf16).
// Kernels, tile choice and launch helpers are in gemm_kernels.h.
#include "gemm_kernels.h"

extern "C" {
int gemm_nt_bf16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                 hipStream_t stream)
{
    const int rc = validate(A, B, D, M, N, K);
    if (rc != GEMM_OK)
        return rc;
    if (M == 0 || N == 0)
        return GEMM_OK;
    if (K == 0) {
        const int64_t count = M * N;
        const int64_t blocks = cdiv(count, 256) < 4096 ? cdiv(count, 256) : 4096;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (uint16_t *)D, count);
    } else {
        launch_plain<false, true>(choose_tile(M, N, K), A, B, D, (int)M, (int)N, (int)K, stream);
    }
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ELAUNCH;
}

} // extern "C"
