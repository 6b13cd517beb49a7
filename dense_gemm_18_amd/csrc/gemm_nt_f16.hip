// gemm_nt_f16.hip -- dense fp16 "NT" GEMM for AMD MI355X (gfx950, CDNA4).
//
//   D[m,n] = sum_k A[m,k] * B[n,k]      A: M x K, B: N x K, D: M x N, fp16
//
// Operation, storage types (fp16 in and out, fp32 accumulator) and the
// NT layout follow page "构建 Tiled GEMM" ("Building a Tiled GEMM", mlc.ai
// modern-gpu-programming-for-mlsys, chapter gemm_basics), section "GEMM".
// The kernel design is gfx950's own; what it keeps from the pages is listed
// next to each part.
//
// One workgroup computes one BM x BN output tile:
//   * Tile -> workgroup map: an XCD-aware remap (consecutive workgroup ids
//     land on different XCDs, each with its own L2) followed by grouped
//     rasterisation, so tiles that share A rows or B rows run on one XCD.
//     Page 2's step 3 ("第 3 步：空间 Tiling（Multi-CTA）", section
//     "Grid 映射") maps the grid straight onto tiles with no reuse between
//     blocks; page 1 ("内核 4：生产级调优") notes that a larger M tile
//     improves L2 reuse of B.
//   * Global -> LDS staging: A and B are both K-contiguous, so one loader
//     serves both.  Each lane moves 16-byte chunks (8 fp16 along K) with
//     buffer loads; 8 lanes cover one 128-byte row of a K-step, so the
//     accesses are fully coalesced (page 1, "内核 1：共享内存分块", shows
//     the cooperative coalesced tile copy).  The buffer resource of each
//     workgroup spans only its valid rows, so rows past M or N read as zero
//     in hardware; K tails are masked per load.
//   * LDS layout: rows of 64 fp16 (128 B = eight 16-byte chunks), chunk index
//     XOR-swizzled by the row so that both the row-wise writer and the
//     column-wise MFMA fragment reader are free of bank conflicts (page 1,
//     "为什么 swizzle 重要", explains the conflict the swizzle removes).
//     Two stages: the loads for K-step k+1 are in flight while the MFMAs of
//     step k run (page 1, "内核 4", double buffering with STAGES = 2).
//   * MFMA: v_mfma_f32_32x32x16_f16, fp32 accumulators in registers.  The B
//     tile is fed as the instruction's first operand and the A tile as its
//     second, so each lane's accumulators hold 4 consecutive columns n of D
//     for one row m and the epilogue writes 8-byte vectors.
//   * Epilogue: fp32 -> fp16 with v_cvt_f16_f32 (round to nearest even),
//     masked at the M and N edges.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_nt_f16.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;            // K elements per LDS row: 128 B, 8 chunks
constexpr int kGroupM = 4;         // tile rows per rasterisation group
constexpr int kXcds = 8;           // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr uint32_t kOob = 0x80000000u;   // a buffer offset past every range
constexpr int kRsrcFlags = 0x00020000;   // gfx9 buffer descriptor word 3

// ---------------------------------------------------------------------------
// Tile -> workgroup map (shared by the kernels and the host introspection).
__host__ __device__ inline void tile_coord(int64_t wg, int64_t tiles_m, int64_t tiles_n,
                                           int64_t &tm, int64_t &tn)
{
    const int64_t total = tiles_m * tiles_n;
    // Hardware deals workgroup ids round-robin over the XCDs; give every XCD
    // a contiguous range of logical ids.
    const int64_t q = total / kXcds, r = total % kXcds;
    const int64_t x = wg % kXcds, i = wg / kXcds;
    const int64_t logical = x * q + (x < r ? x : r) + i;
    // Grouped rasterisation: kGroupM tile rows at a time, rows fastest.
    const int64_t per_group = (int64_t)kGroupM * tiles_n;
    const int64_t g = logical / per_group;
    const int64_t first_m = g * kGroupM;
    const int64_t rows = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
    const int64_t within = logical - g * per_group;
    tm = first_m + within % rows;
    tn = within / rows;
}

// Swizzle of the 16-byte chunk index inside a 128-byte LDS row.  Any 8
// consecutive rows take 8 distinct chunks, and so do the 8 even and the 8
// odd rows among any 16 consecutive ones: a column of 16 B per row read by
// consecutive lanes touches every bank once, whether the LDS serves 128 or
// 256 bytes per clock.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// ---------------------------------------------------------------------------
// Tile configuration.
template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int THREADS = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;      // wave tile
    static constexpr int TM = WTM / 32, TN = WTN / 32;      // MFMA blocks per wave
    static constexpr int CA = BM * 8 / THREADS;             // A chunks per thread per K-step
    static constexpr int CB = BN * 8 / THREADS;
    static constexpr int STAGE = (BM + BN) * kBK;           // fp16 elements per LDS stage
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 MFMA blocks");
    static_assert((BM * 8) % THREADS == 0 && (BN * 8) % THREADS == 0, "chunks must split evenly");
    static_assert(THREADS % 8 == 0, "8 lanes per LDS row");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU");
};

// Load one chunk (8 fp16 along K) of a row panel.  `off` is the byte offset
// of the chunk's first element, `k` its K index.  LOADB is the width of one
// load: 16 (K % 8 == 0, 16-byte aligned panel), 4 (K even, 4-byte aligned)
// or 2 (anything).  Elements with k >= K read as zero; rows past the panel's
// valid rows lie past the buffer range and read as zero in hardware.
template <int LOADB>
__device__ __forceinline__ u32x4 load_chunk(__amdgpu_buffer_rsrc_t rs, uint32_t off, int k, int K)
{
    u32x4 v;
    if constexpr (LOADB == 16) {
        v = __builtin_amdgcn_raw_buffer_load_b128(rs, k < K ? off : kOob, 0, 0);
    } else if constexpr (LOADB == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, k + 2 * j < K ? off + 4 * j : kOob, 0, 0);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                rs, k + 2 * j < K ? off + 4 * j : kOob, 0, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                rs, k + 2 * j + 1 < K ? off + 4 * j + 2 : kOob, 0, 0);
            v[j] = lo | (hi << 16);
        }
    }
    return v;
}

template <class C, int LOADB>
__global__ void __launch_bounds__(C::THREADS, 1)
gemm_nt_f16_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B,
                   _Float16 *__restrict__ D, int M, int N, int K,
                   int tiles_m, int tiles_n, int vec_store)
{
    __shared__ __attribute__((aligned(16))) _Float16 smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % C::WM, wn = wave / C::WM;

    int64_t tm64, tn64;
    tile_coord(blockIdx.x, tiles_m, tiles_n, tm64, tn64);
    const int m0 = (int)tm64 * C::BM, n0 = (int)tn64 * C::BN;
    const int rows_a = min(C::BM, M - m0), rows_b = min(C::BN, N - n0);

    // Buffer resources spanning only this tile's valid rows.
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A + (int64_t)m0 * K), (short)0, rows_a * K * 2, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(B + (int64_t)n0 * K), (short)0, rows_b * K * 2, kRsrcFlags);

    // Loader mapping: thread t moves chunk (t & 7) of rows (t >> 3) + i * THREADS/8.
    const int lrow = tid >> 3, lch = tid & 7;
    constexpr int ROWS_PER_PASS = C::THREADS / 8;
    const uint32_t row_bytes = (uint32_t)K * 2;

    u32x4 stA[C::CA], stB[C::CB];
    auto load_tiles = [&](int k0) {
        const int k = k0 + lch * 8;
#pragma unroll
        for (int i = 0; i < C::CA; ++i)
            stA[i] = load_chunk<LOADB>(ra, (uint32_t)(lrow + i * ROWS_PER_PASS) * row_bytes + (uint32_t)k * 2, k, K);
#pragma unroll
        for (int i = 0; i < C::CB; ++i)
            stB[i] = load_chunk<LOADB>(rb, (uint32_t)(lrow + i * ROWS_PER_PASS) * row_bytes + (uint32_t)k * 2, k, K);
    };
    auto store_tiles = [&](int stage) {
        _Float16 *sa = smem + stage * C::STAGE;
        _Float16 *sb = sa + C::BM * kBK;
#pragma unroll
        for (int i = 0; i < C::CA; ++i) {
            const int row = lrow + i * ROWS_PER_PASS;
            *(u32x4 *)(sa + row * kBK + ((lch ^ swz(row)) << 3)) = stA[i];
        }
#pragma unroll
        for (int i = 0; i < C::CB; ++i) {
            const int row = lrow + i * ROWS_PER_PASS;
            *(u32x4 *)(sb + row * kBK + ((lch ^ swz(row)) << 3)) = stB[i];
        }
    };

    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            acc[i][j] = f32x16{};

    // MFMA fragment rows of this lane (same pattern for A and B: both are
    // K-contiguous).  Lane l supplies row l % 32 and K chunk 2s + l / 32 of
    // each 16-wide K slice s.
    const int frow = lane & 31, fhi = lane >> 5;
    const int a_row0 = wm * C::WTM + frow;
    const int b_row0 = wn * C::WTN + frow;
    const int fsw = swz(frow);   // rows differ from frow by multiples of 32

    auto compute = [&](int stage) {
        const _Float16 *sa = smem + stage * C::STAGE;
        const _Float16 *sb = sa + C::BM * kBK;
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            const int ch = ((2 * s + fhi) ^ fsw) << 3;
            f16x8 af[C::TM], bf[C::TN];
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
                af[i] = *(const f16x8 *)(sa + (a_row0 + 32 * i) * kBK + ch);
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                bf[j] = *(const f16x8 *)(sb + (b_row0 + 32 * j) * kBK + ch);
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
    };

    const int nk = (K + kBK - 1) / kBK;
    load_tiles(0);
    store_tiles(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more)
            load_tiles((kt + 1) * kBK);
        compute(cur);
        if (more)
            store_tiles(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  With B as the MFMA's first operand, accumulator r of block
    // (i, j) holds D[m][n] for m = row base + lane % 32 and
    // n = column base + 8 * (r / 4) + 4 * (lane / 32) + r % 4.
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        const int m = m0 + wm * C::WTM + 32 * i + frow;
        if (m >= M)
            continue;
        _Float16 *drow = D + (int64_t)m * N;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * C::WTN + 32 * j + 8 * g + 4 * fhi;
                f16x4 h;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[r] = (_Float16)acc[i][j][4 * g + r];
                if (vec_store) {
                    if (n < N)
                        *(f16x4 *)(drow + n) = h;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            drow[n + r] = h[r];
                }
            }
        }
    }
}

// D = +0 everywhere (K == 0).
__global__ void fill_zero_kernel(uint16_t *__restrict__ D, int64_t count)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        D[i] = 0;
}

// ---------------------------------------------------------------------------
// Host side.
using Big = Cfg<256, 256, 2, 2>;     // 4 waves, 128 x 128 per wave
using Mid = Cfg<128, 128, 2, 2>;     // 4 waves, 64 x 64 per wave
using Thin = Cfg<64, 64, 2, 2>;      // 4 waves, 32 x 32 per wave

enum class Tile { kBig, kMid, kThin };

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

Tile choose_tile(int64_t M, int64_t N)
{
    if (cdiv(M, 256) * cdiv(N, 256) >= 256)
        return Tile::kBig;
    if (M <= 64 || N <= 64)
        return Tile::kThin;
    return Tile::kMid;
}

void tile_dims(Tile t, int &bm, int &bn)
{
    switch (t) {
    case Tile::kBig: bm = Big::BM; bn = Big::BN; break;
    case Tile::kMid: bm = Mid::BM; bn = Mid::BN; break;
    default: bm = Thin::BM; bn = Thin::BN; break;
    }
}

int validate(const void *A, const void *B, const void *D, int64_t M, int64_t N, int64_t K)
{
    const int64_t lim = INT32_MAX;
    if (M < 0 || N < 0 || K < 0 || M > lim || N > lim || K > GEMM_MAX_K)
        return GEMM_EINVAL;
    const uint64_t a_bytes = (uint64_t)M * (uint64_t)K * 2u;
    const uint64_t b_bytes = (uint64_t)N * (uint64_t)K * 2u;
    const uint64_t d_bytes = (uint64_t)M * (uint64_t)N * 2u;
    if ((a_bytes && !A) || (b_bytes && !B) || (d_bytes && !D))
        return GEMM_EINVAL;
    if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)D) & 1u)
        return GEMM_EINVAL;
    auto overlap = [](const void *p, uint64_t pn, const void *q, uint64_t qn) {
        const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
        return pn && qn && a < b + qn && b < a + pn;
    };
    if (overlap(D, d_bytes, A, a_bytes) || overlap(D, d_bytes, B, b_bytes))
        return GEMM_EINVAL;
    return GEMM_OK;
}

template <class C, int LOADB>
void launch_cfg(const void *A, const void *B, void *D, int M, int N, int K, int vec, hipStream_t s)
{
    const int tm = (int)cdiv(M, C::BM), tn = (int)cdiv(N, C::BN);
    hipLaunchKernelGGL((gemm_nt_f16_kernel<C, LOADB>), dim3((unsigned)(tm * tn)), dim3(C::THREADS),
                       0, s, (const _Float16 *)A, (const _Float16 *)B, (_Float16 *)D, M, N, K,
                       tm, tn, vec);
}

template <class C>
void launch_tile(const void *A, const void *B, void *D, int M, int N, int K, hipStream_t s)
{
    const uintptr_t ab = (uintptr_t)A | (uintptr_t)B;
    const int vec = (((uintptr_t)D & 7u) == 0 && N % 4 == 0) ? 1 : 0;
    if (K % 8 == 0 && (ab & 15u) == 0)
        launch_cfg<C, 16>(A, B, D, M, N, K, vec, s);
    else if (K % 2 == 0 && (ab & 3u) == 0)
        launch_cfg<C, 4>(A, B, D, M, N, K, vec, s);
    else
        launch_cfg<C, 2>(A, B, D, M, N, K, vec, s);
}

} // namespace

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
        switch (choose_tile(M, N)) {
        case Tile::kBig: launch_tile<Big>(A, B, D, (int)M, (int)N, (int)K, stream); break;
        case Tile::kMid: launch_tile<Mid>(A, B, D, (int)M, (int)N, (int)K, stream); break;
        default: launch_tile<Thin>(A, B, D, (int)M, (int)N, (int)K, stream); break;
        }
    }
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ELAUNCH;
}

const char *gemm_nt_f16_strerror(int code)
{
    switch (code) {
    case GEMM_OK: return "success";
    case GEMM_EINVAL: return "invalid argument (size out of range, NULL, misaligned or overlapping pointer)";
    case GEMM_ELAUNCH: return "kernel launch failed";
    default: return "unknown error code";
    }
}

int gemm_nt_f16_tile(int64_t M, int64_t N, int64_t K, int *bm, int *bn, int *bk, int64_t *workgroups)
{
    if (M < 0 || N < 0 || K < 0 || !bm || !bn || !bk || !workgroups)
        return GEMM_EINVAL;
    tile_dims(choose_tile(M, N), *bm, *bn);
    *bk = kBK;
    *workgroups = (M == 0 || N == 0 || K == 0) ? 0 : cdiv(M, *bm) * cdiv(N, *bn);
    return GEMM_OK;
}

int gemm_nt_f16_tile_coord(int64_t wg, int64_t tiles_m, int64_t tiles_n, int64_t *tile_m,
                           int64_t *tile_n)
{
    if (tiles_m <= 0 || tiles_n <= 0 || wg < 0 || wg >= tiles_m * tiles_n || !tile_m || !tile_n)
        return GEMM_EINVAL;
    tile_coord(wg, tiles_m, tiles_n, *tile_m, *tile_n);
    return GEMM_OK;
}

} // extern "C"
