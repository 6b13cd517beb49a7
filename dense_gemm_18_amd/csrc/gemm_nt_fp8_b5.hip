// gemm_nt_fp8_b5.hip -- launches of the FP8 GEMM with B in E5M2 (A in
// either format).  Kernels and helpers: gemm_kernels.h, gemm_fp8.h.
#include "gemm_fp8.h"

void gemm18_fp8_launch_b5(int f8, const void *A, const void *B, void *D, int64_t M, int64_t N,
                          int64_t K, float scale, const float *col_scale, hipStream_t s)
{
    if (f8 == 3)
        launch_fp8<3>(A, B, D, M, N, K, scale, col_scale, s);
    else
        launch_fp8<4>(A, B, D, M, N, K, scale, col_scale, s);
}
