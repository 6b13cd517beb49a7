// gemm_fp8.h -- FP8 launch helpers shared by the two translation units of
// gemm_nt_fp8 (split by B's format so that they compile in parallel).
//
//   D[m,n] = scale * sum_k A[m,k] * B[n,k]     A, B: OCP E4M3 or E5M2 bytes,
//                                               D: fp16, fp32 accumulation
//   (or scale * col_scale[n] per column: per-channel weight scales)
//
// FP8 operands with a per-tensor scale kept in fp32 and applied in the
// epilogue follow the GEMM-optimisation article at www.lqnn.cn (news/123226),
// sections 2.2 (the E4M3 and E5M2 formats) and 4.2-4.3 (quantisation scale,
// fp32 accumulation).  The product runs on the 16-bit direct-to-LDS pipeline
// with FP8 operands seen as 2-byte units (gemm_kernels.h) and the gfx950
// f8f6f4 MFMA; the scale is the fused epilogue's alpha.
#pragma once

#include "gemm_kernels.h"

// Launches the product for format pair F8 = 1 + fa + 2 * fb with fb = 1 (B in
// E5M2); defined in gemm_nt_fp8_b5.hip.  Not exported from the library.
__attribute__((visibility("hidden"))) void gemm18_fp8_launch_b5(
    int f8, const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, float scale,
    const float *col_scale, hipStream_t s);

namespace {


// 128 x 128 tile for FP8: the 16-bit mid tile's pipeline with each step's
// loads issued after the barrier (an FP8 step is a single MFMA slice).
using Mid8 = DmaCfg<128, 128, 2, 2, 64, 4, 16, 16, false>;
// With more 128 x 128 tiles than CUs: two 32 KB stages, two workgroups per
// CU (as Mid2Dma for 16-bit operands).  Measured on MI355X (TFLOP/s, two
// stages / four): 2048 x 4096 x 4096 2081 / 1803, 2560^2 x 4096 1789 / 1486,
// 2304^2 x 8192 1861 / 1670, 3072 x 2048 x 8192 2052 / 1890; at 256 tiles
// (2048^2 x 4096, one workgroup per CU) 1427 / 1859, so the four-stage tile
// keeps those.
using Mid82 = DmaCfg<128, 128, 2, 2, 64, 2, 16, 16, false>;
// 4-byte loads (K % 4 == 0, operands 4-byte aligned): 32 load instructions
// per step, so two stages keep the waits encodable.
using Mid84 = DmaCfg<128, 128, 2, 2, 64, 2, 16, 4, false>;

template <class C, int F8>
void launch_fp8_dma(const void *A, const void *B, void *D, int M, int N, int Kp, int vec,
                    hipStream_t s, const Epi &epi)
{
    using T = _Float16;
    const int tm = (int)cdiv(M, C::BM), tn = (int)cdiv(N, C::BN);
    const SkPlan none{};
    auto go = [&](auto ktail, auto ntc) {
        hipLaunchKernelGGL((gemm_nt_dma_kernel<C, decltype(ktail)::value, false, true, false, F8, 2,
                                               decltype(ntc)::value>),
                           tile_grid((int64_t)tm * tn), dim3(C::THREADS), 0, s, (const T *)A,
                           (const T *)B, (T *)D, M, N, Kp, tm, tn, vec, none, epi);
    };
    // As for 16-bit operands: an operand read once per call (one tile row:
    // B; one tile column: A) streams with the non-temporal policy.
    auto go_nt = [&](auto ktail) {
        if constexpr (C::BM <= 128 && C::LB == 16) {
            switch ((tn == 1 ? 1 : 0) | (tm == 1 ? 2 : 0)) {
            case 1: go(ktail, std::integral_constant<int, 1>{}); return;
            case 2: go(ktail, std::integral_constant<int, 2>{}); return;
            case 3: go(ktail, std::integral_constant<int, 3>{}); return;
            default: break;
            }
        }
        go(ktail, std::integral_constant<int, 0>{});
    };
    if (Kp % C::BK == 0)
        go_nt(std::false_type{});
    else
        go_nt(std::true_type{});
}

// Everything else (K % 4 != 0, or operands not 4-byte aligned): 16-byte
// chunks loaded into registers at any alignment and written to LDS, with K
// counted in bytes (the 128 x 128 or 64 x 64 tile: the 256 x 256 tile's FP8
// fragments leave no registers for the staging).
template <class C, int F8>
void launch_fp8_reg(const void *A, const void *B, void *D, int M, int N, int K, int vec,
                    hipStream_t s, const Epi &epi)
{
    using T = _Float16;
    const int tm = (int)cdiv(M, C::BM), tn = (int)cdiv(N, C::BN);
    const SkPlan none{};
    if (K % C::ROW_BYTES == 0)
        hipLaunchKernelGGL((gemm_nt_dma_kernel<C, false, false, true, false, F8, 1>),
                           tile_grid((int64_t)tm * tn), dim3(C::THREADS), 0, s, (const T *)A,
                           (const T *)B, (T *)D, M, N, K, tm, tn, vec, none, epi);
    else
        hipLaunchKernelGGL((gemm_nt_dma_kernel<C, true, false, true, false, F8, 1>),
                           tile_grid((int64_t)tm * tn), dim3(C::THREADS), 0, s, (const T *)A,
                           (const T *)B, (T *)D, M, N, K, tm, tn, vec, none, epi);
}

// Bytes each lane moves per direct-to-LDS load for FP8 operands with K
// bytes per row: 16, 4, or 0 (register staging).  The 16-byte loads take
// rows that start 16-byte aligned and, as for 16-bit operands, rows that
// start 2-byte aligned (K even, operands 2-byte aligned) on shapes with
// M, N > 64 and at least eight byte pairs per row (the kernel then counts K
// in byte pairs, and the first K-step's chunk that holds k = 0 is rewritten
// from registers).
int fp8_load_bytes(const void *A, const void *B, int64_t M, int64_t N, int64_t K)
{
    const uintptr_t ab = (uintptr_t)A | (uintptr_t)B;
    if (K % 16 == 0 && (ab & 15u) == 0)
        return 16;
    if (K % 2 == 0 && (ab & 1u) == 0 && K >= 16 && M > 64 && N > 64)
        return 16;
    if (K % 4 == 0 && (ab & 3u) == 0)
        return 4;
    return 0;
}

// Tile of the FP8 product: the 16-bit choice on K / 2 byte pairs for 16-byte
// loads (an FP8 step moves the same bytes and does twice the MFMA work);
// with 4-byte loads or register staging the 128 x 128 tile (the 256 x 256
// one would need more loads in flight than the wait counter encodes, or
// more registers) or the thin one.
Tile fp8_tile(int64_t M, int64_t N, int64_t K, int lb)
{
    if (lb == 16)
        return choose_tile(M, N, K / 2, false);
    return (M <= 64 || N <= 64) ? Tile::kThin : Tile::kMid;
}

template <int F8>
void launch_fp8(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                float scale, const float *col_scale, hipStream_t s)
{
    const Epi epi{nullptr, nullptr, scale, 0.0f, col_scale};
    const int lb = fp8_load_bytes(A, B, M, N, K);
    const int vec = store_mode(D, N);
    const int m = (int)M, n = (int)N, kp = (int)(K / 2);
    const Tile t = fp8_tile(M, N, K, lb);
    if (lb == 0) {
        if (t == Tile::kMid)
            launch_fp8_reg<MidReg, F8>(A, B, D, m, n, (int)K, vec, s, epi);
        else
            launch_fp8_reg<ThinReg, F8>(A, B, D, m, n, (int)K, vec, s, epi);
        return;
    }
    if (lb == 16) {
        switch (t) {
        case Tile::kBig: launch_fp8_dma<BigDma, F8>(A, B, D, m, n, kp, vec, s, epi); break;
        case Tile::kMid:
            if (cdiv(M, 128) * cdiv(N, 128) > kCUs)
                launch_fp8_dma<Mid82, F8>(A, B, D, m, n, kp, vec, s, epi);
            else
                launch_fp8_dma<Mid8, F8>(A, B, D, m, n, kp, vec, s, epi);
            break;
        default: launch_fp8_dma<ThinDma, F8>(A, B, D, m, n, kp, vec, s, epi); break;
        }
    } else if (t == Tile::kMid) {
        launch_fp8_dma<Mid84, F8>(A, B, D, m, n, kp, vec, s, epi);
    } else {
        launch_fp8_dma<ThinDma4, F8>(A, B, D, m, n, kp, vec, s, epi);
    }
}

} // namespace
