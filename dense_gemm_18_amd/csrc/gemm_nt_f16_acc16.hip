// gemm_nt_f16_acc16.hip -- C entry points of the fp16 GEMM with an fp16
// running sum (gemm_nt_f16_acc16) and its introspection.
//
//   D[m,n] = s after the last chunk, s <- fp16(s + fp16(sum of the chunk's
//            A[m,k] * B[n,k])), chunks of 64 consecutive k aligned to K's end
//
// The f16 accumulator of page "如何用 Croqtile 一步步优化矩阵乘法内核"
// (sections "内核 0：朴素版", "内核 2：Hopper TMA + WGMMA"), which takes half
// the accumulator registers of fp32.  The product runs on the direct-to-LDS
// (or register-staged) pipeline of gemm_kernels.h with whole-step fragments
// and mma_acc16 as the block update.
#include "gemm_kernels.h"

namespace {

// Tiles.  The fp16 sums fit in the arch VGPRs (the AGPRs stay empty), so at
// least two waves share each SIMD: the block update's VALU work of one wave
// then issues while another's MFMAs run.  256 x 256 with 8 waves of 128 x 64
// (one workgroup per CU); 128 x 128 with 8 waves of 64 x 32, two 32 KB stages
// (two workgroups per CU) when there are more such tiles than CUs, four
// stages (one per CU) otherwise; 64 x 64 for skinny shapes.  Measured on
// MI355X (TFLOP/s): 8192^3 1218-1236 on 256 x 256 (the fp32-accumulating
// kernel: 1481), 1034 on 128 x 128; 4096 x 2048 x 4096 1000 on 128 x 128 with
// 8 waves against 927 with 4 waves of 64 x 64 and 927 on 256 x 256; with at
// most 256 tiles 8 waves and four stages against 4 waves and two: 2048^3 796
// / 581, 1792^2 x 8192 850 / 563, 2048 x 1024 x 4096 586 / 358.  With one wave
// per SIMD (4 waves of 128 x 128 on 256 x 256) the kernel ran 550-600.
using H16Big = DmaCfg<256, 256, 2, 4, 64, 2, 16, 16, false>;
using H16Mid = DmaCfg<128, 128, 2, 4, 64, 2, 16, 16, false>;
using H16Mid4 = DmaCfg<128, 128, 2, 4, 64, 4, 16, 16, false>;
using H16Thin = DmaCfg<64, 64, 2, 2, 64, 8, 16, 16, false>;
// Register-staged 16-byte chunks (K < 8, or skinny shapes whose rows are not
// 16-byte aligned); 128 x 128 at 825 TFLOP/s on 8192^3 with aligned operands.
using H16MidReg = DmaCfg<128, 128, 2, 2, 64, 2, 16, 16, false, true>;
using H16ThinReg = DmaCfg<64, 64, 2, 2, 64, 2, 16, 16, false, true>;

// Tile choice: the smaller (waves of workgroups) x (time per wave), in units
// of the time one CU takes for a 128 x 128 x K tile at the measured rates: a
// wave of 256 x 256 tiles costs 4 / 1218, a wave of up to 256 128 x 128 tiles
// (one per CU) 1 / 850 and a wave of twice 256 (two per CU) 2 / 1034.
// Skinny shapes (M or N at most 64) take 64 x 64.
Tile acc16_tile(int64_t M, int64_t N, bool direct)
{
    if (M <= 64 || N <= 64)
        return Tile::kThin;
    if (!direct)
        return Tile::kMid;
    const int64_t mid_tiles = cdiv(M, 128) * cdiv(N, 128);
    const double big = (double)cdiv(cdiv(M, 256) * cdiv(N, 256), kCUs) * 4.0 / 1218.0;
    const double mid = mid_tiles <= kCUs ? 1.0 / 850.0
                                         : (double)cdiv(mid_tiles, 2 * kCUs) * 2.0 / 1034.0;
    return big <= mid ? Tile::kBig : Tile::kMid;
}

template <class C>
void launch_acc16(const void *A, const void *B, void *D, int M, int N, int K, hipStream_t s)
{
    using T = _Float16;
    const int tm = (int)cdiv(M, C::BM), tn = (int)cdiv(N, C::BN);
    const int vec = store_mode(D, N);
    const SkPlan none{};
    auto go = [&](auto ktail, auto ntc) {
        hipLaunchKernelGGL((gemm_nt_dma_kernel<C, decltype(ktail)::value, false, false, false, 0, 2,
                                               decltype(ntc)::value, true>),
                           tile_grid((int64_t)tm * tn), dim3(C::THREADS), 0, s, (const T *)A,
                           (const T *)B, (T *)D, M, N, K, tm, tn, vec, none, NoEpi{});
    };
    // An operand read once per call (one tile row: B; one tile column: A)
    // streams with the non-temporal policy, as on the other paths.
    auto go_nt = [&](auto ktail) {
        if constexpr (C::BM <= 128 && !C::REG) {
            switch ((tn == 1 ? 1 : 0) | (tm == 1 ? 2 : 0)) {
            case 1: go(ktail, std::integral_constant<int, 1>{}); return;
            case 2: go(ktail, std::integral_constant<int, 2>{}); return;
            case 3: go(ktail, std::integral_constant<int, 3>{}); return;
            default: break;
            }
        }
        go(ktail, std::integral_constant<int, 0>{});
    };
    if (K % C::BK == 0)
        go_nt(std::false_type{});
    else
        go_nt(std::true_type{});
}

void acc16_dims(Tile t, int &bm, int &bn)
{
    switch (t) {
    case Tile::kBig: bm = H16Big::BM; bn = H16Big::BN; break;
    case Tile::kMid: bm = H16Mid::BM; bn = H16Mid::BN; break;
    default: bm = H16Thin::BM; bn = H16Thin::BN; break;
    }
}

} // namespace

extern "C" {
int gemm_nt_f16_acc16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
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
        return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ELAUNCH;
    }
    const bool direct = load_bytes(A, B, M, N, K) == 16;
    const int m = (int)M, n = (int)N, k = (int)K;
    switch (acc16_tile(M, N, direct)) {
    case Tile::kBig: launch_acc16<H16Big>(A, B, D, m, n, k, stream); break;
    case Tile::kMid:
        if (direct && cdiv(M, 128) * cdiv(N, 128) <= kCUs)
            launch_acc16<H16Mid4>(A, B, D, m, n, k, stream);
        else if (direct)
            launch_acc16<H16Mid>(A, B, D, m, n, k, stream);
        else
            launch_acc16<H16MidReg>(A, B, D, m, n, k, stream);
        break;
    default:
        if (direct)
            launch_acc16<H16Thin>(A, B, D, m, n, k, stream);
        else
            launch_acc16<H16ThinReg>(A, B, D, m, n, k, stream);
        break;
    }
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ELAUNCH;
}

int gemm_nt_f16_acc16_kernel(const void *A, const void *B, int64_t M, int64_t N, int64_t K,
                             int *bm, int *bn, int *lbytes)
{
    if (!sizes_ok(M, N, K) || !bm || !bn || !lbytes)
        return GEMM_EINVAL;
    const bool direct = load_bytes(A, B, M, N, K) == 16;
    *lbytes = direct ? 16 : 1;
    acc16_dims(acc16_tile(M, N, direct), *bm, *bn);
    return GEMM_OK;
}
} // extern "C"
