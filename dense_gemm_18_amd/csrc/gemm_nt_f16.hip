// gemm_nt_f16.hip -- C entry points of the fp16 GEMM: gemm_nt_f16, its
// stream-K form and the host-only introspection.
// Kernels, tile choice and launch helpers are in gemm_kernels.h.
#include "gemm_kernels.h"

extern "C" {
int gemm_nt_f16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
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
        launch_plain(choose_tile(M, N, K), A, B, D, (int)M, (int)N, (int)K, stream);
    }
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ELAUNCH;
}

const char *gemm_nt_f16_strerror(int code)
{
    switch (code) {
    case GEMM_OK: return "success";
    case GEMM_EINVAL: return "invalid argument (size out of range, NULL, misaligned or overlapping pointer)";
    case GEMM_ELAUNCH: return "kernel launch failed";
    case GEMM_ESCRATCH: return "the call needs more scratch memory than the library's static buffer holds";
    default: return "unknown error code";
    }
}

int gemm_nt_f16_tile(int64_t M, int64_t N, int64_t K, int *bm, int *bn, int *bk, int64_t *workgroups)
{
    if (!sizes_ok(M, N, K) || !bm || !bn || !bk || !workgroups)
        return GEMM_EINVAL;
    // the load mode of 16-byte aligned operands (load_bytes)
    const bool direct = K % 8 == 0 || (K >= 8 && M > 64 && N > 64);
    tile_dims(run_tile(choose_tile(M, N, K), direct), *bm, *bn);
    *bk = kBK;
    *workgroups = (M == 0 || N == 0 || K == 0) ? 0 : cdiv(M, *bm) * cdiv(N, *bn);
    return GEMM_OK;
}

int gemm_nt_f16_kernel(const void *A, const void *B, const void *D, int64_t M, int64_t N,
                       int64_t K, int *bm, int *bn, int *lbytes, int *store)
{
    if (!sizes_ok(M, N, K) || !bm || !bn || !lbytes || !store)
        return GEMM_EINVAL;
    *lbytes = load_bytes(A, B, M, N, K) == 16 ? 16 : 1;
    tile_dims(run_tile(choose_tile(M, N, K), *lbytes == 16), *bm, *bn);
    *store = store_mode(D, N);
    return GEMM_OK;
}

int gemm_nt_f16_tile_coord(int64_t wg, int64_t tiles_m, int64_t tiles_n, int64_t *tile_m,
                           int64_t *tile_n)
{
    if (tiles_m <= 0 || tiles_n <= 0 || tiles_m > INT32_MAX || tiles_n > INT32_MAX || wg < 0 ||
        wg >= tiles_m * tiles_n || !tile_m || !tile_n)
        return GEMM_EINVAL;
    tile_coord(wg, tiles_m, tiles_n, *tile_m, *tile_n);
    return GEMM_OK;
}

int64_t gemm_nt_f16_ws_size(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || M > INT32_MAX || N > INT32_MAX || K > GEMM_MAX_K)
        return 0;
    const int lb = K >= 8 ? 16 : 0;
    return workspace_bytes(make_plan(M, N, K, lb, kCUs));
}

int gemm_nt_f16_ws(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                   void *workspace, int64_t ws_bytes, hipStream_t stream)
{
    const int rc = validate(A, B, D, M, N, K);
    if (rc != GEMM_OK)
        return rc;
    if (ws_bytes < 0 || (ws_bytes > 0 && !workspace) || ((uintptr_t)workspace & 255u))
        return GEMM_EINVAL;
    if (ws_bytes > 0) {
        const uintptr_t w = (uintptr_t)workspace;
        auto hits = [&](const void *p, int64_t bytes) {
            const uintptr_t q = (uintptr_t)p;
            return bytes > 0 && w < q + (uint64_t)bytes && q < w + (uint64_t)ws_bytes;
        };
        if (hits(A, M * K * 2) || hits(B, N * K * 2) || hits(D, M * N * 2))
            return GEMM_EINVAL;
    }
    const int lb = load_bytes(A, B, M, N, K);
    if (M == 0 || N == 0 || K == 0 || lb == 0)
        return gemm_nt_f16(A, B, D, M, N, K, stream);
    const Plan pl = make_plan(M, N, K, lb, device_cus());
    const int64_t need = workspace_bytes(pl);
    if (!pl.sk || need > ws_bytes)
        return gemm_nt_f16(A, B, D, M, N, K, stream);
    SkPlan sp = pl.split;
    bind_workspace(sp, workspace, pl.grid);
    launch_sk(A, B, D, (int)M, (int)N, (int)K, stream, sp, pl.grid, pl.tile);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ELAUNCH;
}

int gemm_nt_f16_ws_tile(int64_t M, int64_t N, int64_t K, int *bm, int *bn, int64_t *workgroups,
                        int64_t *sk_tiles)
{
    if (!sizes_ok(M, N, K) || !bm || !bn || !workgroups || !sk_tiles)
        return GEMM_EINVAL;
    const int lb = K >= 8 ? 16 : 0;
    const Plan pl = make_plan(M, N, K, (M && N && K) ? lb : 0, kCUs);
    tile_dims(pl.tile, *bm, *bn);
    *sk_tiles = pl.sk ? pl.split.sk_tiles : 0;
    *workgroups = (M == 0 || N == 0 || K == 0) ? 0 : (pl.sk ? pl.grid : cdiv(M, *bm) * cdiv(N, *bn));
    return GEMM_OK;
}

int gemm_nt_f16_ws_items(int64_t M, int64_t N, int64_t K, int64_t wg, int64_t *items,
                         int64_t max_items, int64_t *count)
{
    if (M <= 0 || N <= 0 || K <= 0 || M > INT32_MAX || N > INT32_MAX || K > GEMM_MAX_K ||
        max_items < 0 || (max_items && !items) || !count)
        return GEMM_EINVAL;
    const int lb = K >= 8 ? 16 : 0;
    const Plan pl = make_plan(M, N, K, lb, kCUs);
    *count = 0;
    if (!pl.sk)
        return GEMM_OK;
    if (wg < 0 || wg >= pl.grid)
        return GEMM_EINVAL;
    const int nk = (int)cdiv(K, 64);
    SkCursor cur = sk_begin(pl.split, (int)wg);
    SkItem it;
    while (sk_next(pl.split, nk, pl.grid, cur, it)) {
        if (*count < max_items) {
            int64_t *o = items + 5 * *count;
            o[0] = it.tile;
            o[1] = it.s0;
            o[2] = it.s1;
            o[3] = it.w_first;
            o[4] = it.w_last;
        }
        ++*count;
    }
    return GEMM_OK;
}

} // extern "C"
