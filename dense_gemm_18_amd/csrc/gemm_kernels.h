// gemm_kernels.h -- kernels and host-side planning of the dense "NT" GEMM
// library for AMD MI355X (gfx950, CDNA4), shared by the translation units
// that define the C entry points (one per entry-point family, compiled in
// parallel).  Everything here has internal linkage.
//
//   D[m,n] = sum_k A[m,k] * B[n,k]      A: M x K, B: N x K, D: M x N, fp16
//
// Operation, storage types (fp16 in and out, fp32 accumulator) and the
// NT layout follow page "构建 Tiled GEMM" ("Building a Tiled GEMM", mlc.ai
// modern-gpu-programming-for-mlsys, chapter gemm_basics), section "GEMM".
// The same kernels also serve bfloat16 storage, FP8 operands (2-byte units,
// see mfma_f8), an fp16 running sum (mma_acc16) and the fused
// alpha/beta/bias epilogue.  The kernel design is gfx950's own; what it keeps
// from the pages is listed next to each part.
//
// One workgroup computes one BM x BN output tile (256 x 256, 256 x 128,
// 128 x 128, 64 x 64, 64 x 32 or 32 x 64, by choose_tile); the stream-K form
// instead runs one workgroup per CU over K-step ranges of tile-starved
// shapes and sums split tiles through a workspace (make_plan, sk_next):
//   * Tile -> workgroup map: an XCD-aware remap (consecutive workgroup ids
//     land on different XCDs, each with its own L2) followed by grouped
//     rasterisation, so tiles that share A rows or B rows run on one XCD.
//     Page 2's step 3 ("第 3 步：空间 Tiling（Multi-CTA）", section
//     "Grid 映射") maps the grid straight onto tiles with no reuse between
//     blocks; page 1 ("内核 4：生产级调优") notes that a larger M tile
//     improves L2 reuse of B.
//   * Global -> LDS staging: A and B are both K-contiguous, so one loader
//     serves both.  Each lane moves 16-byte chunks (8 fp16 along K); 8 lanes
//     cover one 128-byte row of a K-step, so the accesses are fully
//     coalesced (page 1, "内核 1：共享内存分块", shows the cooperative
//     coalesced tile copy).  The chunks go straight to LDS (buffer loads
//     that write LDS), also where rows start only 2-byte aligned (odd K,
//     K % 8 != 0, operands offset by whole elements); for K < 8, and for
//     skinny shapes with such rows, they are loaded into registers and
//     written to the same LDS bytes.  The buffer resource of each workgroup
//     spans only its valid rows, so rows past M or N read as zero in
//     hardware; with a K tail the K-steps are aligned to K's end, so only the
//     first step's loads carry a K mask (and, when K % 8 != 0, each row's
//     chunk that holds k = 0 is rewritten from registers).
//   * LDS layout: rows of 64 fp16 (128 B = eight 16-byte chunks), chunk index
//     XOR-swizzled by the row so that the MFMA fragment reader is free of
//     bank conflicts (page 1, "为什么 swizzle 重要", explains the conflict
//     the swizzle removes).  A ring of stages keeps the loads for later
//     K-steps in flight while the MFMAs of the current one run (page 1,
//     "内核 4", double buffering with STAGES = 2).
//   * MFMA: v_mfma_f32_16x16x32_f16 (32x32x16 in the register-staged
//     256 x 256 configuration), fp32 accumulators in registers (or fp16
//     running sums updated once per K-step).  The B tile is fed as the instruction's
//     first operand and the A tile as its second, so each lane's
//     accumulators hold 4 consecutive columns n of D for one row m and the
//     epilogue writes 8-byte vectors.
//   * Epilogue: fp32 -> fp16 with v_cvt_f16_f32 (round to nearest even),
//     masked at the M and N edges, or staged through the freed LDS stages
//     into whole-line stores for tiles wholly inside D; the fused form loads
//     C and bias first and forms alpha * acc + beta * C + bias in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "gemm_nt_f16.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Element type of A, B and D: fp16, or bfloat16 (BF).  Both are 2 bytes,
// so loads, LDS layout and swizzle are shared; the MFMA, the fragment vector
// type and the fp32 -> storage conversion (round to nearest even) differ.
template <bool BF>
struct Elem {
    using T = _Float16;
    using x8 = f16x8;
    using x4 = f16x4;
};
template <>
struct Elem<true> {
    using T = __bf16;
    using x8 = bf16x8;
    using x4 = bf16x4;
};
template <class T>
struct Vec4 {
    using type = f16x4;
};
template <>
struct Vec4<__bf16> {
    using type = bf16x4;
};

template <bool BF>
__device__ __forceinline__ f32x4 mfma16(typename Elem<BF>::x8 b, typename Elem<BF>::x8 a, f32x4 c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c, 0, 0, 0);
}

template <bool BF>
__device__ __forceinline__ f32x16 mfma32(typename Elem<BF>::x8 b, typename Elem<BF>::x8 a,
                                         f32x16 c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c, 0, 0, 0);
}

// FP8 operands (OCP E4M3 or E5M2, one format per operand): F8 = 1 + fa +
// 2 * fb with fa, fb the formats of A and B (0: E4M3, 1: E5M2, the codes of
// the f8f6f4 MFMA's format fields); F8 = 0 for 16-bit operands.  The MFMA is
// v_mfma_f32_16x16x128_f8f6f4 (32 bytes of K per lane and operand, no
// block scales: the per-tensor scale is applied in the epilogue).  B is the
// first operand as in mfma16; any assignment of K bytes to lanes gives the
// same sum as long as A and B use the same one, which they do.
template <int F8>
__device__ __forceinline__ f32x4 mfma_f8(i32x8 b, i32x8 a, f32x4 c)
{
    constexpr int fa = (F8 - 1) & 1, fb = (F8 - 1) >> 1;
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, fb, fa, 0, 0, 0, 0);
}

// fp16 accumulation (page "如何用 Croqtile 一步步优化矩阵乘法内核": an f16
// accumulator, sections "内核 0：朴素版" and "内核 2：Hopper TMA + WGMMA"):
// one 64-wide K-step of a 16x16 block.  CDNA4's MFMAs accumulate in fp32
// only: the step's two 16x16x32 MFMAs sum its 64 products in fp32 from +0,
// the sum is rounded to fp16 (to nearest even) and added to the fp16
// running sum s with a packed fp16 addition, s <- fp16(s + fp16(step sum)).
// Four VALU instructions per block and step (two conversions of pairs, two
// packed adds); widening s into the MFMA's fp32 addend instead would take
// six, and with one wave per SIMD already issuing the MFMAs the VALU issue
// slots are what bounds this kernel.  b and a hold the lane's two 8-element
// K groups of the step (the first for the step's first 32 K).
// The kernel issues the two halves separately (mma_chunk16, then
// acc16_add one block later), so that a block's conversions and adds run
// under the next block's MFMAs instead of waiting for its own.
__device__ __forceinline__ f32x4 mma_chunk16(i32x8 b, i32x8 a)
{
    const f16x8 b0 = __builtin_bit_cast(f16x8, __builtin_shufflevector(b, b, 0, 1, 2, 3));
    const f16x8 b1 = __builtin_bit_cast(f16x8, __builtin_shufflevector(b, b, 4, 5, 6, 7));
    const f16x8 a0 = __builtin_bit_cast(f16x8, __builtin_shufflevector(a, a, 0, 1, 2, 3));
    const f16x8 a1 = __builtin_bit_cast(f16x8, __builtin_shufflevector(a, a, 4, 5, 6, 7));
    f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(b0, a0, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0,
                                                     0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(b1, a1, c, 0, 0, 0);
}

__device__ __forceinline__ f16x4 acc16_add(f16x4 s, f32x4 c)
{
    return s + __builtin_convertvector(c, f16x4);
}

__device__ __forceinline__ f16x4 mma_acc16(i32x8 b, i32x8 a, f16x4 s)
{
    return acc16_add(s, mma_chunk16(b, a));
}

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

// Fused epilogue of gemm_nt_f16_ex: the four consecutive columns n .. n+3
// of row m become alpha * v + beta * C[m][n..] + bias[n..], formed in fp32
// in that order.  beta == 0: C is not read; bias == nullptr: no bias.
// Columns >= N are never read.  vec: C and bias are 8-byte aligned and
// N % 4 == 0 (the same condition as D's vector stores).
struct Epi {
    const _Float16 *C;
    const _Float16 *bias;
    float alpha, beta;
    // FP8 only: N per-column scales; column n is scaled by alpha * col_scale[n]
    // (formed in fp32) instead of alpha.  Null everywhere else.
    const float *col_scale;
};

// Four values of row p at columns n .. n+3 as fp32; columns >= N read as 0
// and are never accessed.  vec: one 8-byte load (N % 4 == 0 and n % 4 == 0,
// so the four columns are all valid or all past the end).
__device__ __forceinline__ f32x4 load4(const _Float16 *p, int n, int N, int vec)
{
    f32x4 v;
    if (vec) {
        const f16x4 h = n < N ? *(const f16x4 *)(p + n) : f16x4{};
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v[r] = (float)h[r];
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v[r] = n + r < N ? (float)p[n + r] : 0.0f;
    }
    return v;
}

struct EpiFin {
    Epi e;
    int N, vec;
    __device__ __forceinline__ f32x4 operator()(f32x4 v, int m, int n) const
    {
        v = v * e.alpha;
        if (e.beta != 0.0f)
            v = v + e.beta * load4(e.C + (int64_t)m * N, n, N, vec);
        if (e.bias)
            v = v + load4(e.bias, n, N, vec);
        return v;
    }
};

struct NoFin {
    __device__ __forceinline__ f32x4 operator()(f32x4 v, int, int) const { return v; }
};

// Kernels without the fused epilogue take this empty argument instead.
struct NoEpi {
};
template <bool EPI>
using EpiArg = typename std::conditional<EPI, Epi, NoEpi>::type;

// Epilogue shared by the kernels.  With B as the MFMA's first operand,
// accumulator r of MFMA block (i, j) holds D[m][n] for
//   m = mbase + 32 i + lane % 32,  n = nbase + 32 j + 8 (r / 4) + 4 (lane / 32) + r % 4,
// so each group of four accumulators is four consecutive columns of one row.
// fp32 -> fp16 uses v_cvt_f16_f32 (round to nearest even); stores are masked
// at the M and N edges.  vec_store: D is 8-byte aligned and N % 4 == 0.
template <int TM, int TN, class T, class Get, class Fin = NoFin>
__device__ __forceinline__ void store_blocks(Get get, T *__restrict__ D, int M, int N,
                                             int mbase, int nbase, int lane, int vec_store,
                                             Fin fin = Fin{})
{
    using X4 = typename Vec4<T>::type;
    const int frow = lane & 31, fhi = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = mbase + 32 * i + frow;
        T *drow = D + (int64_t)m * N;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const f32x16 v = get(i, j);
            if (m >= M)
                continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = nbase + 32 * j + 8 * g + 4 * fhi;
                const f32x4 u = fin(f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]}, m, n);
                X4 h;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    h[r] = (T)u[r];
                if (vec_store) {
                    if (n < N)
                        *(X4 *)(drow + n) = h;
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

template <int TM, int TN, class T>
__device__ __forceinline__ void store_acc(const f32x16 (&acc)[TM][TN], T *__restrict__ D,
                                          int M, int N, int mbase, int nbase, int lane,
                                          int vec_store)
{
    store_blocks<TM, TN>([&](int i, int j) { return acc[i][j]; }, D, M, N, mbase, nbase, lane,
                         vec_store);
}

// Staged epilogue of a wave's (16 TM) x (16 TN) output tile: the 16-bit
// results are first written to the wave's own LDS buffer, rows of 32 TN
// bytes whose 16-byte chunks are XOR-swizzled by the row (conflict-free for
// the 16-rows-by-8-bytes writes of one MFMA block), then read back along
// rows and written to D with 16-byte stores, each instruction covering whole
// 128-byte lines of consecutive rows.  Written straight from the MFMA layout,
// one store covers 32 bytes of each of 16 rows; when every CU finishes a
// tile at once (the lock-step waves of a large GEMM) those partial-line
// stores take several microseconds to drain, the staged ones about a third.
// Used for tiles wholly inside D, with D 16-byte aligned and N % 8 == 0.
template <int TM, int TN>
struct Stage16 {
    static constexpr int CPR = 2 * TN;            // 16-byte chunks per row
    static constexpr int ROWB = 32 * TN;
    static constexpr int BYTES = 16 * TM * ROWB;
    // byte offset of the 8-byte group of columns n .. n+3 (n % 4 == 0) of row r
    __device__ static int offset(int r, int n)
    {
        return r * ROWB + (((n >> 3) ^ (r % CPR)) << 4) + ((n >> 2) & 1) * 8;
    }
};

// Read a wave's staged tile back row by row and store it at dtile (row
// pitch N elements).  The caller's writes to `stage` are this wave's own, and
// LDS operations of one wave complete in order.
template <int TM, int TN, class T>
__device__ __forceinline__ void flush_stage16(const char *stage, T *__restrict__ dtile, int N,
                                              int lane)
{
    using S = Stage16<TM, TN>;
    constexpr int RPI = 64 / S::CPR;              // rows per instruction
    static_assert(64 % S::CPR == 0 && (16 * TM) % RPI == 0, "whole rows per instruction");
    const int c = lane % S::CPR, r0 = lane / S::CPR;
    T *dp = dtile + 8 * c;
#pragma unroll
    for (int it = 0; it < 16 * TM / RPI; ++it) {
        const int r = it * RPI + r0;
        const u32x4 v = *(const u32x4 *)(stage + r * S::ROWB + ((c ^ (r % S::CPR)) << 4));
        *(u32x4 *)(dp + (int64_t)r * N) = v;
    }
}

// Same for v_mfma_f32_16x16x32_f16 blocks (B as the first operand):
// accumulator r of block (i, j) holds D[m][n] for
//   m = mbase + 16 i + lane % 16,  n = nbase + 16 j + 4 (lane / 16) + r.
// STAGED: the tile lies wholly inside D (no row or column checks) and its
// groups go to the wave's staging buffer `stage` (flushed by the caller)
// instead of D.
template <int TM, int TN, class T, class Get, class Fin = NoFin, bool STAGED = false>
__device__ __forceinline__ void store_blocks16(Get get, T *__restrict__ D, int M, int N,
                                               int mbase, int nbase, int lane, int vec_store,
                                               Fin fin = Fin{}, char *stage = nullptr)
{
    using X4 = typename Vec4<T>::type;
    const int frow = lane & 15, fq = lane >> 4;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = mbase + 16 * i + frow;
        T *drow = D + (int64_t)m * N;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const f32x4 v = get(i, j);
            if constexpr (!STAGED) {
                if (m >= M)
                    continue;
            }
            const int n = nbase + 16 * j + 4 * fq;
            const f32x4 u = fin(v, m, n);
            X4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                h[r] = (T)u[r];
            if constexpr (STAGED) {
                *(u32x2 *)(stage + Stage16<TM, TN>::offset(16 * i + frow, 16 * j + 4 * fq)) =
                    __builtin_bit_cast(u32x2, h);
            } else if (vec_store) {
                if (n < N)
                    *(X4 *)(drow + n) = h;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N)
                        drow[n + r] = h[r];
            }
        }
    }
}

// Four fp16 values of row p at columns n .. n+3 (columns >= N read as 0),
// raw: one 8-byte load when vec, else element loads.
__device__ __forceinline__ f16x4 load4h(const _Float16 *p, int n, int N, int vec)
{
    if (vec)
        return n < N ? *(const f16x4 *)(p + n) : f16x4{};
    f16x4 h;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        h[r] = n + r < N ? p[n + r] : (_Float16)0.0f;
    return h;
}

// The fused epilogue on 16x16 blocks (same element map as store_blocks16)
// in two phases: every C and bias value this lane needs is loaded first (in
// registers as fp16, 2 VGPRs per group of four), then each group becomes
// alpha * v + beta * C + bias in fp32 in that order and is stored.  All the
// loads are in flight together instead of one load latency per group.
// WITH_C / WITH_BIAS = false: the caller has established that C (beta == 0)
// or the bias is absent, which keeps their registers and code out (the FP8
// kernels, whose epilogue is a scale alone).  COLS: e.col_scale is present
// (FP8 with per-channel scales; the caller branches on it once, so that no
// form computes the other's arithmetic).
template <int TM, int TN, class Get, bool WITH_C = true, bool COLS = false, bool WITH_BIAS = true,
          bool STAGED = false>
__device__ __forceinline__ void store_blocks16_epi(Get get, _Float16 *__restrict__ D, int M,
                                                   int N, int mbase, int nbase, int lane,
                                                   int vec, const Epi &e, char *stage = nullptr)
{
    const int frow = lane & 15, fq = lane >> 4;
    const bool has_c = WITH_C && e.beta != 0.0f, has_bias = WITH_BIAS && e.bias != nullptr;
    f16x4 cv[TM][TN], bv[TN];
    // per-column factors alpha * col_scale[n .. n+3] (columns >= N not read)
    f32x4 sv[COLS ? TN : 1];
    if constexpr (COLS) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = nbase + 16 * j + 4 * fq;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sv[j][r] = e.alpha * (n + r < N ? e.col_scale[n + r] : 0.0f);
        }
    }
    if (has_bias) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bv[j] = load4h(e.bias, nbase + 16 * j + 4 * fq, N, vec);
    }
    if (has_c) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = mbase + 16 * i + frow;
#pragma unroll
            for (int j = 0; j < TN; ++j)
                cv[i][j] = m < M ? load4h(e.C + (int64_t)m * N, nbase + 16 * j + 4 * fq, N, vec)
                                 : f16x4{};
        }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = mbase + 16 * i + frow;
        _Float16 *drow = D + (int64_t)m * N;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const f32x4 v = get(i, j);
            if constexpr (!STAGED) {
                if (m >= M)
                    continue;
            }
            const int n = nbase + 16 * j + 4 * fq;
            f32x4 u;
            if constexpr (COLS)
                u = v * sv[j];
            else
                u = v * e.alpha;
            if (has_c) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    u[r] = u[r] + e.beta * (float)cv[i][j][r];
            }
            if (has_bias) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    u[r] = u[r] + (float)bv[j][r];
            }
            f16x4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                h[r] = (_Float16)u[r];
            if constexpr (STAGED) {
                *(u32x2 *)(stage + Stage16<TM, TN>::offset(16 * i + frow, 16 * j + 4 * fq)) =
                    __builtin_bit_cast(u32x2, h);
            } else if (vec) {
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

template <int TM, int TN, class T>
__device__ __forceinline__ void store_acc16(const f32x4 (&acc)[TM][TN], T *__restrict__ D,
                                            int M, int N, int mbase, int nbase, int lane,
                                            int vec_store)
{
    store_blocks16<TM, TN>([&](int i, int j) { return acc[i][j]; }, D, M, N, mbase, nbase, lane,
                           vec_store);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS kernel (fast path: K % 8 == 0, A and B 16-byte aligned).
//
// gfx950's buffer_load_dwordx4 ... lds writes each lane's 16 bytes straight
// into LDS, at M0 + 16 * lane: one instruction fills 1024 contiguous bytes
// and needs no staging registers and no ds_write.  That leaves room for a
// ring of NSTAGE LDS stages of BK = 64, so the loads for later K-steps are
// in flight while step u is multiplied (page 1, "内核 3：Warp 特化" and
// "内核 4", overlaps loads with MMAs through a STAGES-deep ring; here one
// wavefront both loads and multiplies, and the ring is tracked with vmcnt
// and one workgroup barrier per K-step instead of full/empty events).
//
// LDS rows are BK 2-byte elements (BK = 64 in every configuration: 128
// bytes, eight 16-byte chunks; the template also takes BK = 32).  The
// swizzle is applied on the global side: LDS slot (row, chunk) receives
// global chunk chunk ^ swz_row(row) of that row.  The swizzles were chosen
// by measuring SQ_LDS_BANK_CONFLICT for the MFMA fragment read patterns
// (16 or 32 rows x 16 bytes per group of lanes) on gfx950: zero conflicts.

typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS buffer load of LB bytes per lane.  The size is spelled as a
// literal in each branch: the builtin's host-side check of a dependent size
// argument rejects 16 (a gfx950-only width) and silently drops the kernel.
// AUX: the cache-policy bits (kNt: non-temporal).
constexpr int kNt = 2;
template <int LB, int AUX = 0>
__device__ __forceinline__ void load_lds(__amdgpu_buffer_rsrc_t rs, char *dst, uint32_t voff,
                                         uint32_t soff)
{
    if constexpr (LB == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, voff, soff, 0, AUX);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 4, voff, soff, 0, AUX);
}

// The eight 16-bit elements of v moved up by s places (s in 1..7, uniform
// across the wave): element j of the result is element j - s of v, and
// elements 0 .. s-1 are zero.
__device__ __forceinline__ u32x4 shift_up_halves(u32x4 v, int s)
{
    const uint64_t lo = (uint64_t)v[0] | ((uint64_t)v[1] << 32);
    const uint64_t hi = (uint64_t)v[2] | ((uint64_t)v[3] << 32);
    const int b = 16 * s;
    uint64_t nlo, nhi;
    if (b < 64) {
        nlo = lo << b;
        nhi = (hi << b) | (lo >> (64 - b));
    } else {
        nlo = 0;
        nhi = lo << (b - 64);
    }
    return u32x4{(uint32_t)nlo, (uint32_t)(nlo >> 32), (uint32_t)nhi, (uint32_t)(nhi >> 32)};
}

__device__ __forceinline__ int swz64(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// 128-byte rows read by 16x16x32 fragments (16 rows x 16 bytes per quarter
// wave): measured conflict-free, and also for the 32x32x16 pattern.
__device__ __forceinline__ int swz128_q(int row) { return (row >> 1) & 7; }

// Chunk swizzle of an LDS row of BK fp16 read by MF x MF MFMA fragments.
template <int BK, int MF>
__device__ __forceinline__ int swz_row(int row)
{
    return BK == 64 ? (MF == 32 ? swz(row) : swz128_q(row)) : swz64(row);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt
// left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Kernel-local lambdas must always inline: an out-of-line call would keep
// every array they capture by reference in scratch memory.
#define G18_INLINE __attribute__((always_inline))

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E-1, so that
// register arrays are only ever indexed by constants.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Workgroup barrier without a memory fence (a fence would wait for every
// outstanding direct-to-LDS load, prefetches included).  This wave's LDS
// reads complete first (lgkmcnt 0, issued as the builtin so the compiler's
// own wait tracking sees it); the empty asm with a "memory" clobber keeps
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int BM_, int BN_, int WM_, int WN_, int BK_, int NSTAGE_, int MF_, int LB_, bool SPLIT_,
          bool REG_ = false, bool B3_ = false>
struct DmaCfg {
    // B3: B gets a ring of three stages while A keeps two (two 32 KB A
    // stages and three 32 KB B stages fill the 160 KB of LDS at 256 x 256).
    // B's refills then go out in the first slice of a step, with a step and a
    // half to land, and A's in the second as before: each slice issues half
    // a step's loads instead of one slice issuing all of them.
    static constexpr bool B3 = B3_;
    // LB: bytes one lane moves per load: 16 (buffer_load_dwordx4 ... lds,
    // needs K % 8 == 0 and 16-byte aligned operands) or 4 (buffer_load_dword
    // ... lds, needs K even and 4-byte aligned operands).
    static constexpr int LB = LB_;
    // REG: the same 16-byte chunks, loaded into registers at any alignment
    // (gfx950's vector memory loads take unaligned addresses) and written to
    // LDS with ds_write_b128 at the byte the direct-to-LDS load would fill;
    // serves any K and any 2-byte-aligned operands (used for K < 8, skinny
    // shapes whose rows are not 16-byte aligned, and FP8 rows at any byte
    // alignment).  Each chunk is loaded
    // one step ahead of its LDS write, and the register is reloaded right
    // after the write, so every load has a full step to land wherever the
    // write sits in the step.  The writes of a step are spread evenly over
    // one step's worth of slices: a group in the slice after the barrier
    // that frees their stage, the other groups in the next step's slices
    // before its barrier.
    static constexpr bool REG = REG_;
    // SPLIT: a step's loads are issued half in the slice after the barrier
    // and half in the next step's first slice; otherwise all of them in the
    // slice after the barrier (which gives every load the longest time to
    // land when a step has only two slices).
    static constexpr bool SPLIT = SPLIT_;
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NSTAGE = NSTAGE_;
    static constexpr int BK = BK_;
    // MF = 32: v_mfma_f32_32x32x16_f16; MF = 16: v_mfma_f32_16x16x32_f16.
    static constexpr int MF = MF_;
    static constexpr int KSL = MF == 32 ? 16 : 32;           // K per MFMA (one slice)
    static constexpr int SLICES = BK / KSL;                  // slices per step
    static constexpr int CHS = KSL / 8;                      // 16-byte chunks per slice
    static constexpr int CPR = BK / 8;                       // 16-byte chunks per LDS row
    static constexpr int NWAVES = WM * WN, THREADS = NWAVES * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / MF, TN = WTN / MF;
    using acc_t = typename std::conditional<MF == 32, f32x16, f32x4>::type;
    static constexpr int ROW_BYTES = BK * 2;                 // 64 or 128
    static constexpr int INST_BYTES = 64 * LB;               // LDS bytes one load instruction fills
    static constexpr int ROWS_PER_INST = INST_BYTES / ROW_BYTES;
    static constexpr int LPR = ROW_BYTES / LB;               // lanes per LDS row in one load
    static constexpr int A_LOADS = BM / ROWS_PER_INST / NWAVES;   // per wave per stage
    static constexpr int B_LOADS = BN / ROWS_PER_INST / NWAVES;
    static constexpr int LPS = A_LOADS + B_LOADS;            // vmcnt units per stage
    // Stages: A and B interleaved per stage, or (B3) all A stages then all
    // B stages.  Steps cycle through PERIOD ring positions; a step at
    // position p uses A stage p % NSTAGE and B stage p % NSB.
    static constexpr int NSB = B3 ? NSTAGE + 1 : NSTAGE;
    static constexpr int PERIOD = B3 ? NSTAGE * NSB : NSTAGE;
    static constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;
    static constexpr int LDS_BYTES = NSTAGE * BM * ROW_BYTES + NSB * BN * ROW_BYTES;
    static constexpr int a_base(int s) { return B3 ? s * BM * ROW_BYTES : s * STAGE_BYTES; }
    static constexpr int b_base(int s)
    {
        return B3 ? NSTAGE * BM * ROW_BYTES + s * BN * ROW_BYTES : s * STAGE_BYTES + BM * ROW_BYTES;
    }
    static_assert(MF == 32 || MF == 16, "MFMA block of 32x32 or 16x16");
    static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be whole MFMA blocks");
    static_assert(BM % (ROWS_PER_INST * NWAVES) == 0 && BN % (ROWS_PER_INST * NWAVES) == 0,
                  "load instructions must split evenly over the waves");
    static_assert(BK == 32 || BK == 64, "LDS rows of 64 or 128 bytes");
    static_assert(LB == 16 || LB == 4, "16- or 4-byte loads");
    static_assert(ROWS_PER_INST >= 1, "a load covers whole LDS rows");
    // The largest vmcnt the pipeline waits on (prologue) must be encodable.
    static_assert(NSTAGE >= 2 && LPS * (NSTAGE - 2) + LPS / 2 < 64, "vmcnt budget");
    static_assert(SLICES % 2 == 0, "slice 0 of every step uses fragment set 0");
    static_assert(SPLIT || LPS * (NSTAGE - 1) < 64, "vmcnt budget");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU");
    static_assert(!REG || (LB == 16 && NSTAGE == 2 && BK == 64 && !SPLIT && LPS % SLICES == 0),
                  "register staging: 16-byte chunks, two stages, writes in every slice");
    static_assert(!B3 || (NSTAGE == 2 && !SPLIT && !REG && SLICES == 2 && A_LOADS == B_LOADS),
                  "three B stages: two A stages, two slices, square load split");
};

// Stream-K work split of a persistent grid of P workgroups (one per CU, all
// resident at once).  Tiles [0, dp_tiles) are whole tiles, dealt round-robin
// (dp_tiles is a multiple of P, so every workgroup gets as many).  The K-steps
// of tiles [dp_tiles, dp_tiles + sk_tiles), in tile-major order, are split
// into P contiguous ranges: workgroup w gets base + (w < extra) of them.
// A tile split over several workgroups is finished by its owner, the one that
// runs the tile's first step: every other contributor starts its range inside
// that tile, writes its fp32 partial sums to its own slot and raises its flag;
// the owner adds the slots in ascending workgroup order (so results do not
// depend on timing) and rounds once to fp16.
//
// Flags carry the call's epoch instead of a fixed value, so a flag left by an
// earlier call never reads as raised: every workgroup reads the epoch word
// e at its start and the call uses e + 1 (0 skipped); the last workgroup to
// finish (a done counter) stores e + 1 back and zeroes the counter, ready for
// the next call on the stream.  A zero-filled workspace is a valid start.
struct SkPlan {
    int dp_tiles, sk_tiles;
    int base, extra;
    uint32_t *hdr;        // kSkHdrWords words: epoch, done counter, error word
    uint32_t *flags;      // P words
    float *partials;      // P slots of BM * BN floats
};
// Workspace header: word 0 the last completed call's epoch, word 1 the count
// of workgroups done in the running call (0 between calls), word 2 nonzero
// once an owner gave up waiting for a contributor (sticky; the caller clears
// it).  The header is 256 bytes, followed by the flags and the slots.
constexpr int kSkHdrWords = 64;
constexpr int kSkErrWord = 2;

// One work item of workgroup w: K-steps [s0, s1) of `tile`.  s0 > 0: w is a
// contributor to that tile.  Otherwise w writes the tile, adding the partial
// sums of workgroups w_first .. w_last (none when w_first > w_last).
struct SkItem {
    int tile, s0, s1, w_first, w_last;
};

// Walks workgroup w's items: its whole tiles w, w + P, ... below dp_tiles,
// then the pieces of its stream-K range, each ending at a tile boundary or
// at the range end.  Host and device run the same code (the host to test it).
struct SkCursor {
    int t_dp, i, iend;
};

__host__ __device__ inline int sk_wg_of(const SkPlan &sk, int i)   // the workgroup whose range holds step i
{
    const int cut = sk.extra * (sk.base + 1);
    return i < cut ? i / (sk.base + 1) : sk.extra + (sk.base ? (i - cut) / sk.base : 0);
}

__host__ __device__ inline SkCursor sk_begin(const SkPlan &sk, int w)
{
    const int i = w * sk.base + (w < sk.extra ? w : sk.extra);
    return SkCursor{w, i, i + sk.base + (w < sk.extra ? 1 : 0)};
}

__host__ __device__ inline bool sk_next(const SkPlan &sk, int nk, int P, SkCursor &c, SkItem &it)
{
    it.w_first = 1;
    it.w_last = 0;
    if (c.t_dp < sk.dp_tiles) {
        it.tile = c.t_dp;
        it.s0 = 0;
        it.s1 = nk;
        c.t_dp += P;
        return true;
    }
    if (c.i >= c.iend)
        return false;
    const int j = c.i / nk;
    it.s0 = c.i - j * nk;
    it.s1 = it.s0 + (c.iend - c.i) < nk ? it.s0 + (c.iend - c.i) : nk;
    it.tile = sk.dp_tiles + j;
    c.i += it.s1 - it.s0;
    if (it.s0 == 0 && it.s1 < nk) {
        it.w_first = sk_wg_of(sk, j * nk + it.s1);
        it.w_last = sk_wg_of(sk, j * nk + nk - 1);
    }
    return true;
}

// Polls of a contributor's flag before an owner gives up (~5 s at 1.6 GHz):
// the tile is then written as NaN and the kernel still ends.  Every wave
// polls for itself: the kernel keeps a single LDS object (a second one, to
// broadcast the result, costs the compiler its proof that fragment reads do
// not overlap in-flight direct-to-LDS loads, and it then waits for all of
// them before every read).
constexpr int kSpinLimit = 1 << 24;

// KTAIL: K % BK != 0; the K-steps are then aligned to K's end, so the
// first step starts before k = 0 and only its loads (in the prologue of the
// tile's first work item) carry a per-lane K mask.  SK: the persistent
// stream-K form; otherwise one workgroup per tile.  F8 != 0: FP8 operands
// (see mfma_f8), passed as 2-byte units: K counts byte pairs, so loads, LDS
// layout, swizzle and K masks are those of the 16-bit path.  A K-step (a
// 128-byte row) is one f8f6f4 MFMA per block; its two slices split the
// blocks by rows instead of the K-step by halves.
// UB: bytes of one K unit: 2 (16-bit elements, or FP8 byte pairs), or 1 (FP8
// bytes, register staging only: any K and any alignment).  K counts units;
// a K-step is one 128-byte LDS row, BKU units.  NT (direct-to-LDS loads):
// bit 0 loads A, bit 1 loads B with the non-temporal cache policy, set when
// that operand is read exactly once per call (a single column or row of
// tiles), so that streaming it does not allocate in the caches.  H16: the
// running sum is fp16 (mma_acc16), one update per K-step and block.
template <class C, bool KTAIL, bool SK, bool EPI, bool BF, int F8 = 0, int UB = 2, int NT = 0,
          bool H16 = false>
__global__ void __launch_bounds__(C::THREADS, 1)
gemm_nt_dma_kernel(const typename Elem<BF>::T *__restrict__ A,
                   const typename Elem<BF>::T *__restrict__ B, typename Elem<BF>::T *__restrict__ D,
                   int M, int N, int K, int tiles_m, int tiles_n, int vec_store, SkPlan sk,
                   EpiArg<EPI> epi)
{
    // WIDE: a fragment holds the lane's part of a whole K-step (32 bytes),
    // and each block takes all of a step's products at once: FP8 (one f8f6f4
    // MFMA per step) and fp16 accumulation (both 16x16x32 MFMAs of the step
    // back to back, before the fp16 rounding).  The two slices of a step
    // then split the blocks by rows instead of the K-step by halves.
    constexpr bool WIDE = F8 != 0 || H16;
    using X8 = typename std::conditional<WIDE, i32x8, typename Elem<BF>::x8>::type;
    static_assert(!WIDE || (!BF && !SK && !C::SPLIT && C::MF == 16 && C::BK == 64 &&
                            C::SLICES == 2 && C::NSTAGE % 2 == 0 && C::TM % 2 == 0),
                  "whole-step fragments: 16x16 blocks, 128-byte rows, an even stage ring, "
                  "loads after the barrier");
    static_assert(!WIDE || !C::B3, "whole-step fragments: one ring for A and B");
    static_assert(!H16 || (F8 == 0 && !EPI && UB == 2), "fp16 accumulation: fp16 operands");
    static_assert(UB == 2 || (UB == 1 && F8 != 0 && C::REG), "byte units: FP8, register staging");
    constexpr int BKU = C::ROW_BYTES / UB;      // K units per step
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases in SGPRs
    const int wm = wave % C::WM, wn = wave / C::WM;

    // The current work item: tile origin (m0, n0), buffer resources spanning
    // the tile's valid rows of A and B, and its K-steps [s0, s0 + n).
    int m0 = 0, n0 = 0, kb = 0, n = 0;
    __amdgpu_buffer_rsrc_t ra, rb;
    // Zero-length resource: every load through it reads zero.  Steps past the
    // end of the item use it, chosen per step in scalar registers.
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        (void *)A, (short)0, 0, kRsrcFlags);
    const int nk = (K + BKU - 1) / BKU;
    auto set_item = [&](int64_t tile, int s0, int s1) G18_INLINE {
        int64_t tm64, tn64;
        tile_coord(tile, tiles_m, tiles_n, tm64, tn64);
        m0 = (int)tm64 * C::BM;
        n0 = (int)tn64 * C::BN;
        const int rows_a = min(C::BM, M - m0), rows_b = min(C::BN, N - n0);
        ra = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)A + (int64_t)m0 * K * UB),
                                               (short)0, rows_a * K * UB, kRsrcFlags);
        rb = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)B + (int64_t)n0 * K * UB),
                                               (short)0, rows_b * K * UB, kRsrcFlags);
        // With a K tail the steps are aligned to K's end instead of its
        // start: step 0 covers k in [-shift, BK - shift) and every later
        // step is full, so only the first step's loads need a K mask.
        kb = s0 * BKU - (KTAIL ? nk * BKU - K : 0);
        n = s1 - s0;
    };

    // This lane's part of each load instruction: LDS slot `lane` of a block
    // of ROWS_PER_INST rows is row lane / CPR, chunk lane % CPR; it fetches
    // the global chunk that the swizzle places there.  Instruction i of this
    // wave covers rows ROWS_PER_INST * (wave + NWAVES * i) and up.  The
    // vector offsets carry rows and chunks only; a step's K offset travels in
    // the scalar offset, so a full step issues its loads with no VALU work.
    // With LB = 4 a lane moves one 4-byte quarter of a chunk (intra-chunk
    // byte offset `sub`).
    //
    // These per-lane values, and the fragment addresses below, are set up
    // per work item from `ln`, a copy of the lane id that the compiler must
    // treat as changing: otherwise it keeps them live across the persistent
    // loop's epilogues, where the 256 accumulators leave no registers free.
    uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
    int a_k[C::A_LOADS], b_k[C::B_LOADS];
    // Offset and first k of load q (A's loads first, then B's); only the
    // operand's own array is indexed, since the two have their own lengths.
    auto off_of = [&](auto qc) G18_INLINE {
        constexpr int q = decltype(qc)::value;
        if constexpr (q < C::A_LOADS)
            return a_off[q];
        else
            return b_off[q - C::A_LOADS];
    };
    auto k_of = [&](auto qc) G18_INLINE {
        constexpr int q = decltype(qc)::value;
        if constexpr (q < C::A_LOADS)
            return a_k[q];
        else
            return b_k[q - C::A_LOADS];
    };
    auto setup_loads = [&](int ln) G18_INLINE {
        const int slot_row = ln / C::LPR;
        const int slot_byte = (ln % C::LPR) * C::LB;
        const int sub = slot_byte % 16;
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i) {
            const int row = C::ROWS_PER_INST * (wave + C::NWAVES * i) + slot_row;
            const int gch = (slot_byte / 16) ^ swz_row<C::BK, C::MF>(row);
            a_k[i] = (gch * 16 + sub) / UB;
            a_off[i] = (uint32_t)row * (uint32_t)K * UB + (uint32_t)(gch * 16 + sub);
        }
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
            const int row = C::ROWS_PER_INST * (wave + C::NWAVES * i) + slot_row;
            const int gch = (slot_byte / 16) ^ swz_row<C::BK, C::MF>(row);
            b_k[i] = (gch * 16 + sub) / UB;
            b_off[i] = (uint32_t)row * (uint32_t)K * UB + (uint32_t)(gch * 16 + sub);
        }
    };

    // One global->LDS load q of step `step` into stage S: q < A_LOADS moves
    // A rows, the rest B rows; each instruction fills 1024 contiguous LDS
    // bytes.  Rows past the tile's valid rows lie past the buffer range and
    // read as zero; steps past the end load through the zero-length
    // resource.  FIRST (the prologue's first step only): with a K tail the
    // item's first step may start before k = 0 (k0 < 0, uniform); chunks
    // with k < 0 then get an out-of-range offset and the others carry k0 in
    // their vector offset.  Loads inside the K-loop carry no mask, which
    // keeps the loop's registers those of the untailed kernel.
    // REG: chunk q of the next step to be written to LDS, in registers.  A
    // load puts row 8 (wave + NWAVES i) + lane / 8, global chunk
    // (lane % 8) ^ swizzle into rst[q] (the chunk the direct-to-LDS load
    // would bring), and the write stores it at that load's LDS byte.
    u32x4 rst[C::REG ? C::LPS : 1];
    auto reg_load = [&](int step, auto qc, auto firstc) G18_INLINE {
        constexpr int q = decltype(qc)::value;
        constexpr bool isa = q < C::A_LOADS;
        const int k0 = kb + step * BKU;
        const __amdgpu_buffer_rsrc_t rs = step < n ? (isa ? ra : rb) : rz;
        const uint32_t off = off_of(qc);
        const uint32_t soff = (uint32_t)k0 * (uint32_t)UB;
        if constexpr (KTAIL && decltype(firstc)::value) {
            if (k0 < 0) {
                // The item's first step starts before k = 0: a chunk whose
                // first k is negative reads element by element, k < 0 as
                // zero (such a chunk may start in the row before, or before
                // the buffer).  Offsets wrap modulo 2^32, as soff does.
                const int kk = k0 + k_of(qc);
                if (kk >= 0) {
                    rst[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + soff, 0, 0);
                } else {
                    u32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t o = off + soff + 4u * j;
                        if constexpr (UB == 2) {
                            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                                rs, kk + 2 * j >= 0 ? o : kOob, 0, 0);
                            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                                rs, kk + 2 * j + 1 >= 0 ? o + 2u : kOob, 0, 0);
                            v[j] = lo | (hi << 16);
                        } else {
                            uint32_t w = 0;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(
                                         rs, kk + 4 * j + e >= 0 ? o + e : kOob, 0, 0)
                                     << (8 * e);
                            v[j] = w;
                        }
                    }
                    rst[q] = v;
                }
                return;
            }
        }
        rst[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, soff, 0);
    };
    auto reg_write = [&](auto sc, auto qc) G18_INLINE {
        constexpr int S = decltype(sc)::value, q = decltype(qc)::value;
        constexpr bool isa = q < C::A_LOADS;
        constexpr int i = isa ? q : q - C::A_LOADS;
        constexpr int base = (isa ? C::a_base(S) : C::b_base(S)) + (i * C::NWAVES) * C::INST_BYTES;
        *(u32x4 *)(smem + base + wave * C::INST_BYTES + lane * 16) = rst[q];
    };

    auto issue_one = [&](int step, auto sc, auto qc, auto firstc) G18_INLINE {
        constexpr int S = decltype(sc)::value, q = decltype(qc)::value;
        if constexpr (C::REG) {
            // stage S takes step `step` (already in registers); the registers
            // then load step + 1
            reg_write(sc, qc);
            reg_load(step + 1, qc, std::false_type{});
            return;
        }
        const int k0 = kb + step * BKU;
        const bool live = step < n;
        constexpr bool isa = q < C::A_LOADS;
        // S: the ring position of `step`
        char *stage = smem + (isa ? C::a_base(S % C::NSTAGE) : C::b_base(S % C::NSB));
        constexpr int i = isa ? q : q - C::A_LOADS;
        uint32_t off = off_of(qc);
        uint32_t soff = (uint32_t)k0 * 2u;
        if constexpr (KTAIL && decltype(firstc)::value) {
            if (k0 < 0) {
                const int kk = k_of(qc);
                off = k0 + kk >= 0 ? off + soff : kOob;
                soff = 0;
            }
        }
        char *dst = stage + (wave + C::NWAVES * i) * C::INST_BYTES;
        load_lds<C::LB, (NT >> (isa ? 0 : 1)) & 1 ? kNt : 0>(live ? (isa ? ra : rb) : rz, dst, off,
                                                              soff);
    };

    // Accumulators: fp32 blocks, or (H16) the fp16 running sums, four per
    // lane and 16x16 block in the fp32 layout.
    using AccT = typename std::conditional<H16, f16x4, typename C::acc_t>::type;
    AccT acc[C::TM][C::TN];
    // Block (i, j) in fp32 for the epilogue (exact for fp16 sums).
    auto accf = [&](int i, int j) G18_INLINE {
        if constexpr (H16)
            return __builtin_convertvector(acc[i][j], f32x4);
        else
            return acc[i][j];
    };

    // Fragments of one K slice (16 wide for 32x32x16, 32 wide for 16x16x32):
    // lane l holds row l % MF of each MF-row block and K chunk
    // CHS * t + l / MF of slice t (the same pattern for A and B, which are
    // both K-contiguous).  Fragment q < TM is A block q, the rest B blocks.
    // The LDS address of every (stage, slice) is precomputed, so a fragment
    // read is one ds_read_b128 with an immediate offset.
    uint32_t a_addr[C::NSTAGE][C::SLICES], b_addr[C::NSB][C::SLICES];
    auto setup_reads = [&](int ln) G18_INLINE {
        const int frow = ln % C::MF, fhi = ln / C::MF;
        const int fsw = swz_row<C::BK, C::MF>(frow);   // fragment rows differ from frow by multiples of MF
#pragma unroll
        for (int st = 0; st < C::NSB; ++st)
#pragma unroll
            for (int t = 0; t < C::SLICES; ++t) {
                const uint32_t ch = (uint32_t)(((C::CHS * t + fhi) ^ fsw) * 16);
                if (st < C::NSTAGE)
                    a_addr[st][t] = C::a_base(st) + (wm * C::WTM + frow) * C::ROW_BYTES + ch;
                b_addr[st][t] = C::b_base(st) + (wn * C::WTN + frow) * C::ROW_BYTES + ch;
            }
    };
    // Two fragment sets (alternating slices): A blocks fa[set][i], B blocks
    // fb[set][j].
    X8 fa[2][C::TM], fb[2][C::TN];
    auto frag = [&](auto setc, auto qc) G18_INLINE -> X8 & {
        constexpr int f = decltype(setc)::value, q = decltype(qc)::value;
        if constexpr (q < C::TM)
            return fa[f][q];
        else
            return fb[f][q - C::TM];
    };
    auto read_one = [&](auto setc, auto sc, auto tc, auto qc) G18_INLINE {
        constexpr int S = decltype(sc)::value, t = decltype(tc)::value, q = decltype(qc)::value;
        constexpr int off = C::MF * (q < C::TM ? q : q - C::TM) * C::ROW_BYTES;
        X8 &f = frag(setc, qc);
        if constexpr (WIDE) {
            // 32 bytes: the chunks of both 16-bit slices (t is always 0)
            static_assert(t == 0, "a whole-step fragment spans the K-step");
            const uint32_t p0 = q < C::TM ? a_addr[S][0] : b_addr[S][0];
            const uint32_t p1 = q < C::TM ? a_addr[S][1] : b_addr[S][1];
            const u32x4 lo = *(const u32x4 *)(smem + p0 + off);
            const u32x4 hi = *(const u32x4 *)(smem + p1 + off);
            f = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            f = *(const X8 *)(smem + (q < C::TM ? a_addr[S % C::NSTAGE][t] : b_addr[S % C::NSB][t]) +
                              off);
        }
    };

    constexpr int NM = C::TM * C::TN, NR = C::TM + C::TN;
    // MFMAs per slice: all blocks, or (FP8) half of the block rows.
    constexpr int NMS = WIDE ? NM / 2 : NM;
    constexpr int LHALF = C::LPS / 2;
    // Loads issued in one slice: half a step's or a whole step's (register
    // staging: a step's writes and reloads over all its slices).
    constexpr int LSL = (C::REG && !WIDE) ? C::LPS / C::SLICES
                        : C::B3           ? C::A_LOADS
                                          : (C::SPLIT ? LHALF : C::LPS);
    // The LSL loads of a slice are spread evenly over its NMS MFMAs (load l
    // after MFMA floor(l NMS / LSL)); RPG fragment reads follow each MFMA.
    constexpr int RPG = (NR + NM - 1) / NM;
    static_assert(C::LPS % 2 == 0, "loads split evenly over the slices that issue them");
    // Whole-step read schedule (FP8, fp16 accumulation), by the slice's MFMA
    // index p: the next step's B
    // blocks (double-buffered) during the first slice, B block j after
    // p = j * BSTEP; its A blocks (single-buffered) during the second: those
    // of the first half-rows (dead since the first slice) after p = 0, 1, ...,
    // A block i of the second half once row i is done with the current one.
    constexpr int HR = C::TM / 2;
    constexpr int BSTEP = NMS / C::TN > 1 ? NMS / C::TN : 1;

    // One slice: MFMA q of TM x TN, each followed by its share of fragment
    // reads for the next slice (stage RS, slice RT) and of the loads l0, l0+1,
    // ... of step lstep into stage LS.  The scheduling fences keep exactly
    // this issue order: with one wavefront per SIMD nothing else fills an
    // issue gap, and the four waves share the CU's load pipe (about 25 cycles
    // per 1 KB load), so loads are spread evenly rather than issued in a burst.
    // Whole-step fragments are twice as large and a K-step's are read in its
    // second slice only; the A fragments are not double buffered (see the
    // whole-step read schedule above), which keeps the 256 x 256 FP8 tile
    // within the registers.
    // h: (whole-step fragments) which half of the block rows this slice
    // multiplies.
    // cur, nxt: fragment sets (integral constants) multiplied and read.
    f32x4 pend;     // (H16) the chunk sum of the block multiplied last
    auto slice = [&](auto cur, auto nxt,
                     auto do_read, auto rs, auto rt, auto do_load, int lstep, auto ls,
                     auto l0, auto hc) G18_INLINE {
        static_for<0, NMS>([&](auto pc) G18_INLINE {
            constexpr int p = decltype(pc)::value;
            constexpr int q = p + (WIDE ? decltype(hc)::value * NMS : 0);
            constexpr int i = q / C::TN, j = q % C::TN;
            using QA = std::integral_constant<int, i>;
            using QB = std::integral_constant<int, C::TM + j>;
            if constexpr (F8 != 0)
                acc[i][j] = mfma_f8<F8>(frag(cur, QB{}), frag(cur, QA{}), acc[i][j]);
            else if constexpr (H16) {
                // this block's chunk sum; the previous block's fp16 update
                // now, under these MFMAs; the slice's last block at its end
                const f32x4 c = mma_chunk16(frag(cur, QB{}), frag(cur, QA{}));
                __builtin_amdgcn_sched_barrier(0);     // both MFMAs first
                if constexpr (p > 0) {
                    constexpr int qp = q - 1;
                    acc[qp / C::TN][qp % C::TN] = acc16_add(acc[qp / C::TN][qp % C::TN], pend);
                }
                pend = c;
                if constexpr (p == NMS - 1)
                    acc[i][j] = acc16_add(acc[i][j], pend);
            }
            else if constexpr (C::MF == 32)
                acc[i][j] = mfma32<BF>(frag(cur, QB{}), frag(cur, QA{}), acc[i][j]);
            else
                acc[i][j] = mfma16<BF>(frag(cur, QB{}), frag(cur, QA{}), acc[i][j]);
            if constexpr (decltype(do_read)::value && WIDE && decltype(hc)::value == 0) {
                static_for<0, C::TN>([&](auto jc) G18_INLINE {
                    constexpr int jb = decltype(jc)::value;
                    constexpr int pb = jb * BSTEP < NMS ? jb * BSTEP : NMS - 1;
                    if constexpr (p == pb)
                        read_one(nxt, rs, rt, std::integral_constant<int, C::TM + jb>{});
                });
            } else if constexpr (decltype(do_read)::value && WIDE) {
                if constexpr (p < HR)
                    read_one(nxt, rs, rt, std::integral_constant<int, p>{});
                if constexpr (j == C::TN - 1)
                    read_one(nxt, rs, rt, std::integral_constant<int, i>{});
            } else if constexpr (decltype(do_read)::value) {
                static_for<q * RPG, (q * RPG + RPG < NR ? q * RPG + RPG : NR)>(
                    [&](auto rc) G18_INLINE { read_one(nxt, rs, rt, rc); });
            }
            // loads ceil(p LSL / NMS) .. ceil((p + 1) LSL / NMS) - 1 after MFMA p
            if constexpr (decltype(do_load)::value)
                static_for<(p * LSL + NMS - 1) / NMS, ((p + 1) * LSL + NMS - 1) / NMS>(
                    [&](auto gc) G18_INLINE {
                        issue_one(lstep, ls,
                                  std::integral_constant<int, decltype(l0)::value +
                                                                  decltype(gc)::value>{},
                                  std::false_type{});
                    });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    using T_ = std::true_type;
    using F_ = std::false_type;
    using Z_ = std::integral_constant<int, 0>;
    using H_ = std::integral_constant<int, LHALF>;

    // Software pipeline over K-steps of BK (SLICES slices each).  Fragments
    // are double-buffered: slice t + 1 is read while slice t is multiplied.
    // Before the last slice of step u, the workgroup barrier makes step u + 1
    // readable and frees step u's stage, which is refilled with step
    // u + NSTAGE: all of its loads during the last slice of step u, or with
    // SPLIT the first half there and the second half during the first slice
    // of step u + 1 (each step's loads stay contiguous in issue order, so
    // "step u + 1 has landed" is "at most (NSTAGE - 2) * LPS loads
    // outstanding").  Step u + 1's first fragments
    // load under the last MFMAs of step u.  Every step, the last included,
    // runs the same code: refills of steps past the end read zeros into
    // stages no one reads again, which keeps the vmcnt accounting the same in
    // every iteration.  S is step u's stage, a compile-time constant: the
    // step loop is unrolled NSTAGE times.
    auto step_body = [&](int u, auto sc) G18_INLINE {
        // S: the ring position of step u (the stage itself unless B3)
        constexpr int S = decltype(sc)::value;
        using S_ = std::integral_constant<int, S>;
        using SP_ = std::integral_constant<int, (S + C::NSTAGE - 1) % C::PERIOD>;   // step u-1+NSTAGE
        using SN_ = std::integral_constant<int, (S + 1) % C::PERIOD>;               // step u+1
        using SR_ = std::integral_constant<int, (S + C::NSTAGE) % C::PERIOD>;       // step u+NSTAGE
        using SB_ = std::integral_constant<int, (S + C::NSB - 1) % C::PERIOD>;      // step u+NSB-1
        if constexpr (WIDE) {
            // Whole-step fragments (FP8, fp16 accumulation): the barrier
            // comes first (step u + 1 landed, step u's stage free); the first
            // slice refills the stage with step u + NSTAGE and reads step
            // u + 1's B blocks, the second reads its A blocks.
            // LDS reads and DMA writes are then spread over the whole step,
            // and each refill still has the step's second slice to land.
            // Both slices multiply fragment set S & 1 (an even ring).
            constexpr int c = S & 1;
            using H1_ = std::integral_constant<int, 1>;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!C::REG)
                wait_vmcnt<C::LPS * (C::NSTAGE - 2)>();
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            slice(std::integral_constant<int, c>{}, std::integral_constant<int, c ^ 1>{}, T_{}, SN_{}, Z_{}, T_{}, u + C::NSTAGE, SR_{}, Z_{}, Z_{});
            slice(std::integral_constant<int, c>{}, std::integral_constant<int, c ^ 1>{}, T_{}, SN_{}, Z_{}, F_{}, 0, S_{}, Z_{}, H1_{});
        } else {
        static_for<0, C::SLICES>([&](auto tc) G18_INLINE {
            constexpr int t = decltype(tc)::value;
            constexpr int c = t & 1;    // 16-bit slices alternate fragment sets
            using TN_ = std::integral_constant<int, t + 1>;
            if constexpr (C::B3 && t == 0) {
                // B's refill: step u + NSB - 1 into the B stage step u - 1
                // left (free since the previous step's barrier)
                slice(std::integral_constant<int, c>{}, std::integral_constant<int, c ^ 1>{}, T_{},
                      S_{}, TN_{}, T_{}, u + C::NSB - 1, SB_{},
                      std::integral_constant<int, C::A_LOADS>{}, tc);
            } else if constexpr (C::REG && t + 1 < C::SLICES) {
                // group t + 1 of step u - 1 + NSTAGE (its stage was freed at
                // the previous step's barrier)
                slice(std::integral_constant<int, c>{}, std::integral_constant<int, c ^ 1>{}, T_{}, S_{}, TN_{}, T_{}, u - 1 + C::NSTAGE, SP_{},
                      std::integral_constant<int, (t + 1) * LSL>{}, tc);
            } else if constexpr (t == 0 && C::SPLIT) {
                // second half of step u - 1 + NSTAGE
                slice(std::integral_constant<int, c>{}, std::integral_constant<int, c ^ 1>{}, T_{}, S_{}, TN_{}, T_{}, u - 1 + C::NSTAGE, SP_{}, H_{}, tc);
            } else if constexpr (t + 1 < C::SLICES) {
                slice(std::integral_constant<int, c>{}, std::integral_constant<int, c ^ 1>{}, T_{}, S_{}, TN_{}, F_{}, 0, S_{}, Z_{}, tc);
            } else {
                // Step u+1 has landed once only steps u+2 .. u+NSTAGE-1 may
                // be outstanding.  The fence keeps the previous slice's MFMAs
                // ahead of the barrier, where they run while the wave waits.
                // (Register staging waits for each chunk's load only before
                // writing it; the compiler places those waits.)
                // (B3: only B's refill for step u + 2, issued in this
                // step's first slice, may be outstanding.)
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (C::B3)
                    wait_vmcnt<C::B_LOADS>();
                else if constexpr (!C::REG)
                    wait_vmcnt<C::LPS * (C::NSTAGE - 2)>();
                lds_barrier();
                __builtin_amdgcn_sched_barrier(0);
                slice(std::integral_constant<int, c>{}, std::integral_constant<int, c ^ 1>{}, T_{}, SN_{}, Z_{}, T_{}, u + C::NSTAGE, SR_{}, Z_{}, tc);
            }
        });
        }
    };
    // acc = the sum over the current item's K-steps (steps are counted from
    // the item's first one).

    // 16x16 blocks of a tile wholly inside D, with D 16-byte aligned and
    // N % 8 == 0 (vec_store == 2), go through LDS (store_blocks16's staged
    // form); with the fused epilogue only for FP8 operands, whose epilogue
    // is the scale alone (beta == 0).  (The 16-bit fused-epilogue kernel keeps
    // the direct stores: next to its C registers the staging code makes the
    // 256 x 256 kernel spill.)  The stages are free once every wave is past its
    // last fragment read and its loads have landed (wait_vmcnt<0> before
    // this, then the barrier); each wave then owns BM * BN * 2 / NWAVES
    // bytes of them.
    auto store_d = [&]() G18_INLINE {
        const int mb = m0 + wm * C::WTM, nb = n0 + wn * C::WTN;
        if constexpr (C::MF == 16 && (!EPI || F8 != 0)) {
            using St = Stage16<C::TM, C::TN>;
            static_assert(St::BYTES * C::NWAVES <= C::LDS_BYTES, "staging fits the LDS stages");
            bool staged = vec_store == 2 && m0 + C::BM <= M && n0 + C::BN <= N;
            if constexpr (EPI)
                staged = staged && epi.beta == 0.0f;
            if (staged) {
                lds_barrier();
                char *stage = smem + wave * St::BYTES;
                auto get = [&](int i, int j) G18_INLINE { return accf(i, j); };
                if constexpr (EPI) {     // FP8: the scale alone, or per-column scales
                    if (epi.col_scale)
                        store_blocks16_epi<C::TM, C::TN, decltype(get), false, true, false, true>(
                            get, D, M, N, mb, nb, lane, vec_store, epi, stage);
                    else
                        store_blocks16_epi<C::TM, C::TN, decltype(get), false, false, false, true>(
                            get, D, M, N, mb, nb, lane, vec_store, epi, stage);
                }
                else
                    store_blocks16<C::TM, C::TN, typename Elem<BF>::T, decltype(get), NoFin, true>(
                        get, D, M, N, mb, nb, lane, vec_store, NoFin{}, stage);
                flush_stage16<C::TM, C::TN>(stage, D + (int64_t)mb * N + nb, N, lane);
                return;
            }
        }
        if constexpr (EPI) {
            auto get = [&](int i, int j) G18_INLINE { return accf(i, j); };
            if constexpr (C::MF == 32)
                store_blocks<C::TM, C::TN>(get, D, M, N, mb, nb, lane, vec_store,
                                           EpiFin{epi, N, vec_store});
            else if constexpr (F8 != 0) {
                if (epi.col_scale)
                    store_blocks16_epi<C::TM, C::TN, decltype(get), false, true, false>(
                        get, D, M, N, mb, nb, lane, vec_store, epi);
                else
                    store_blocks16_epi<C::TM, C::TN, decltype(get), false, false, false>(
                        get, D, M, N, mb, nb, lane, vec_store, epi);
            } else {
                store_blocks16_epi<C::TM, C::TN>(get, D, M, N, mb, nb, lane, vec_store, epi);
            }
        } else if constexpr (C::MF == 32) {
            store_acc<C::TM, C::TN>(acc, D, M, N, mb, nb, lane, vec_store);
        } else if constexpr (H16) {
            store_blocks16<C::TM, C::TN>(accf, D, M, N, mb, nb, lane, vec_store);
        } else {
            store_acc16<C::TM, C::TN>(acc, D, M, N, mb, nb, lane, vec_store);
        }
    };

    // ---- stream-K epilogue helpers ----
    // Hand-off between workgroups on different XCDs, whose L2 caches are not
    // coherent with each other: partial sums and flags move with the sc1
    // cache policy (coherent at device scope, like device-scope atomics), and
    // a contributor's stores are complete (vmcnt 0) before its flag is
    // raised.  No device-scope fence is used: on this part a fence writes
    // back or invalidates a whole L2, which would evict every other
    // workgroup's staged A and B lines.
    constexpr int kSc1 = 16;    // cache-policy bits of a buffer access: sc1
    // A partial slot holds each lane's accumulators in register order, 16
    // bytes per lane per access: piece e of block q of wave v, lane l, is at
    // byte (((v * NM + q) * P4 + e) * 64 + l) * 16, so every access is one
    // fully coalesced 1 KB buffer access whose per-block part is a constant
    // scalar offset (one lane offset in a VGPR for the whole slot).
    constexpr int P4 = (int)(sizeof(typename C::acc_t) / 16);     // 16-byte pieces per block
    auto slot_rsrc = [&](int wslot) G18_INLINE {
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)(sk.partials + (int64_t)wslot * (C::BM * C::BN)), (short)0,
            C::BM * C::BN * 4, kRsrcFlags);
    };
    auto slot_store = [&](__amdgpu_buffer_rsrc_t rs, int voff) G18_INLINE {
        static_for<0, NM>([&](auto qc) G18_INLINE {
            constexpr int q = decltype(qc)::value;
            const auto &a = acc[q / C::TN][q % C::TN];
#pragma unroll
            for (int e = 0; e < P4; ++e) {
                const f32x4 v = {a[4 * e], a[4 * e + 1], a[4 * e + 2], a[4 * e + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, voff,
                                                       (q * P4 + e) * 1024, kSc1);
            }
            __builtin_amdgcn_sched_barrier(0);    // one block at a time: no register peak
        });
    };
    // Owner: add the partial sums of slots w_first .. w_last, in that order.
    // Loads are issued RB blocks at a time (the fragment registers are free
    // here), so one memory latency covers RB KB per wave instead of one.
    constexpr int RB = NM % 16 == 0 ? 16 : NM;
    auto add_partials = [&](int w_first, int w_last, int voff) G18_INLINE {
        for (int w2 = w_first; w2 <= w_last; ++w2) {
            const __amdgpu_buffer_rsrc_t rs = slot_rsrc(w2);
            static_for<0, NM / RB>([&](auto bc) G18_INLINE {
                constexpr int b0 = decltype(bc)::value * RB;
                f32x4 pf[RB][P4];
                static_for<0, RB>([&](auto gc) G18_INLINE {
                    constexpr int q = b0 + decltype(gc)::value;
#pragma unroll
                    for (int e = 0; e < P4; ++e)
                        pf[decltype(gc)::value][e] = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       rs, voff, (q * P4 + e) * 1024, kSc1));
                });
                static_for<0, RB>([&](auto gc) G18_INLINE {
                    constexpr int q = b0 + decltype(gc)::value;
                    auto &a = acc[q / C::TN][q % C::TN];
#pragma unroll
                    for (int e = 0; e < P4; ++e)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            a[4 * e + r] += pf[decltype(gc)::value][e][r];
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        }
    };
    // D for the current tile; ok == false (a contributor never arrived)
    // writes NaN instead.
    auto store_ok = [&](bool ok) G18_INLINE {
        auto get = [&](int bi, int bj) G18_INLINE {
            return ok ? accf(bi, bj) : typename C::acc_t{} + __builtin_nanf("");
        };
        if constexpr (C::MF == 32)
            store_blocks<C::TM, C::TN>(get, D, M, N, m0 + wm * C::WTM, n0 + wn * C::WTN, lane,
                                       vec_store);
        else
            store_blocks16<C::TM, C::TN>(get, D, M, N, m0 + wm * C::WTM, n0 + wn * C::WTN, lane,
                                         vec_store);
    };

    // The work loop: one pass (this workgroup's tile) for the one-tile-per-
    // workgroup form; the persistent form walks its items.  The pipeline is
    // written out here once, not wrapped in a lambda: wrapped, the register
    // allocator moves accumulators and fragments between register files
    // inside the K-loop.
    const int w = blockIdx.x;
    SkCursor cur = sk_begin(sk, w);
    uint32_t epoch = 0;
    if constexpr (SK) {
        const uint32_t e0 = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(sk.hdr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        epoch = e0 + 1u ? e0 + 1u : 1u;
    }
    for (;;) {
        SkItem it{};
        if constexpr (SK) {
            if (!sk_next(sk, nk, gridDim.x, cur, it))
                break;
            lds_barrier();             // every wave is done with the LDS stages
            set_item(it.tile, it.s0, it.s1);
        } else {
            // one tile per workgroup; a grid of more tiles than one grid
            // dimension holds spreads over y, and workgroups past the last
            // tile end here, before any barrier
            const int64_t tile = (int64_t)blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
            if (tile >= (int64_t)tiles_m * tiles_n)
                return;
            set_item(tile, 0, nk);
        }
    int ln = lane;
    asm volatile("" : "+v"(ln));
    setup_loads(ln);
    setup_reads(ln);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            acc[i][j] = AccT{};

    // Prologue: steps 0 .. NSTAGE-2 and, with split loads, the first half of
    // step NSTAGE-1 (its second half is issued by step 0's first slice, like
    // every later step); otherwise all of step NSTAGE-1 too.
    constexpr int PRO_LAST = C::REG ? LSL : (C::SPLIT ? LHALF : C::LPS);
    if constexpr (C::REG) {
        // Steps 0 .. NSTAGE-2 and the first group of step NSTAGE-1 through
        // the registers into their stages; those registers then load step
        // NSTAGE, the others keep step NSTAGE-1's chunks for the slices of
        // step 0 before its barrier.
        static_for<0, C::NSTAGE>([&](auto sc) G18_INLINE {
            constexpr int st = decltype(sc)::value;
            static_for<0, C::LPS>([&](auto qc) G18_INLINE {
                reg_load(st, qc, std::integral_constant<bool, st == 0>{});
            });
            wait_vmcnt<0>();
            static_for<0, (st + 1 < C::NSTAGE ? C::LPS : PRO_LAST)>(
                [&](auto qc) G18_INLINE { reg_write(sc, qc); });
        });
        static_for<0, PRO_LAST>([&](auto qc) G18_INLINE {
            reg_load(C::NSTAGE, qc, std::false_type{});
        });
        lds_barrier();
    } else {
    // With K % 8 != 0 the steps, aligned to K's end, start their 16-byte
    // chunks at k = K mod 8 + 8j, so in the item's first step (k0 < 0) one
    // chunk of each row holds k = -8 + e .. e - 1 with e = K mod 8: 8 - e
    // elements of the row before (or of no row) and the row's first e.  Its
    // direct load, like those of the chunks wholly before k = 0, gets the
    // out-of-range offset and fills zeros; the row's first eight elements
    // are loaded into registers ahead of the stage's direct loads (so the
    // stage's wait covers them), moved up by 8 - e places and written over
    // those zeros before the barrier that publishes the stage.  Rows past
    // the tile's valid rows load zeros.  (Needs K >= 8: a row then spans the
    // 16 bytes read from its start.)
    constexpr bool FIX = KTAIL && UB == 2 && C::LB == 16;
    const int fe = FIX && kb < 0 ? (kb & 7) : 0;       // uniform: K mod 8, or 0
    u32x4 fixv[FIX ? C::LPS : 1];
    auto fix_chunk = [&](auto qc) G18_INLINE -> bool {
        const int kk = kb + k_of(qc);
        return kk < 0 && kk > -8;
    };
    if constexpr (FIX) {
        if (fe != 0) {
            static_for<0, C::LPS>([&](auto qc) G18_INLINE {
                constexpr int q = decltype(qc)::value;
                constexpr bool isa = q < C::A_LOADS;
                if (fix_chunk(qc)) {
                    const uint32_t row0 = off_of(qc) - (uint32_t)(k_of(qc) * 2);
                    fixv[q] = __builtin_amdgcn_raw_buffer_load_b128(n > 0 ? (isa ? ra : rb) : rz,
                                                                    row0, 0, 0);
                }
            });
        }
    }
    static_for<0, C::NSTAGE>([&](auto sc) G18_INLINE {
        constexpr int st = decltype(sc)::value;
        static_for<0, (st + 1 < C::NSTAGE ? C::LPS : PRO_LAST)>(
            [&](auto qc) G18_INLINE {
                issue_one(st, sc, qc, std::integral_constant<bool, st == 0>{});
            });
    });
    wait_vmcnt<C::LPS * (C::NSTAGE - 2) + PRO_LAST>();
    if constexpr (FIX) {
        if (fe != 0) {
            static_for<0, C::LPS>([&](auto qc) G18_INLINE {
                constexpr int q = decltype(qc)::value;
                constexpr bool isa = q < C::A_LOADS;
                constexpr int i = isa ? q : q - C::A_LOADS;
                if (fix_chunk(qc)) {
                    char *dst = smem + (isa ? C::a_base(0) : C::b_base(0)) +
                                (wave + C::NWAVES * i) * C::INST_BYTES + lane * 16;
                    *(u32x4 *)dst = shift_up_halves(fixv[q], 8 - fe);
                }
            });
        }
    }
    lds_barrier();
    }
    static_for<0, NR>([&](auto qc) G18_INLINE { read_one(Z_{}, Z_{}, Z_{}, qc); });

    // With two stages the step count is rounded up to even instead of
    // guarding each step (a guard costs registers at the loop back-edge):
    // an extra step multiplies the all-zero stage that the zero-length
    // resource filled, and adding +0 leaves every accumulator unchanged (an
    // fp32 sum that starts at +0 is never -0).
    for (int u = 0; u < n; u += C::PERIOD)
        static_for<0, C::PERIOD>([&](auto sc) G18_INLINE {
            if (C::PERIOD <= 2 || u + decltype(sc)::value < n)
                step_body(u + decltype(sc)::value, sc);
        });
    wait_vmcnt<0>();      // drain the zero-filling prefetches

        if constexpr (!SK) {
            store_d();
            break;
        } else {
        const int s0 = it.s0;
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int slot_voff = (wave * NM * P4 * 64 + ln) * 16;
        if (s0 > 0) {
            // Contributor: publish the partial sums, then the flag.  The
            // stores are device-coherent (sc1) and complete (vmcnt 0) in
            // every wave before the barrier; the compiler barriers keep the
            // flag store after them in program order.
            slot_store(slot_rsrc(w), slot_voff);
            wait_vmcnt<0>();
            __syncthreads();
            asm volatile("" ::: "memory");
            if (tid == 0)
                __hip_atomic_store(sk.flags + w, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("" ::: "memory");
            continue;
        }
        // Owner of a split tile (or a whole tile: an empty range): wait for
        // the contributors' flags, add their partials, store D.
        const int w_first = it.w_first, w_last = it.w_last;
        bool ok = true;
        if (w_first <= w_last) {
            for (int w2 = w_first; w2 <= w_last && ok; ++w2) {
                int got = 0;
                for (int poll = 0; poll < kSpinLimit; ++poll) {
                    if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                            sk.flags + w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == epoch) {
                        got = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(8);
                }
                ok = got != 0;
            }
        }
        // The slot loads below must not move above the polls: the flag's
        // value is needed (s_waitcnt) before the loop exits, and this
        // compiler barrier keeps the loads after it in program order.
        asm volatile("" ::: "memory");
        if (ok)
            add_partials(w_first, w_last, slot_voff);
        else if (tid == 0)
            __hip_atomic_store(sk.hdr + kSkErrWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        store_ok(ok);
        }
    }
    if constexpr (SK) {
        // The last workgroup to finish publishes the epoch for the next call.
        __syncthreads();
        if (tid == 0) {
            const uint32_t done = __hip_atomic_fetch_add(sk.hdr + 1, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            if (done + 1u == gridDim.x) {
                __hip_atomic_store(sk.hdr + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(sk.hdr, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// K == 0 with the fused epilogue: D = alpha * (+0) + beta * C + bias (with FP8
// column scales, alpha * col_scale[n] in place of alpha).
[[maybe_unused]] __global__ void epilogue_only_kernel(_Float16 *__restrict__ D, Epi e, int64_t M, int64_t N)
{
    const int64_t count = M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const float s = e.col_scale ? e.alpha * e.col_scale[i % N] : e.alpha;
        float v = s * 0.0f;
        if (e.beta != 0.0f)
            v = v + e.beta * (float)e.C[i];
        if (e.bias)
            v = v + (float)e.bias[i % N];
        D[i] = (_Float16)v;
    }
}

// D = +0 everywhere (K == 0).
[[maybe_unused]] __global__ void fill_zero_kernel(uint16_t *__restrict__ D, int64_t count)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        D[i] = 0;
}

// ---------------------------------------------------------------------------
// Host side.
// 256 x 256: 4 waves of 128 x 128 on 16x16x32 MFMAs, two 64 KB stages, each
// step's loads issued right after the barrier.  16x16x32 keeps half as many
// accumulator registers busy per FLOP as 32x32x16, so the part draws less
// power and holds a higher clock under its power limit.
using BigDma = DmaCfg<256, 256, 2, 2, 64, 2, 16, 16, false>;
// The same tile with three B stages (two 32 KB A stages, three 32 KB B
// stages: the whole 160 KB), for K % 512 != 0.  B's refills then go out in
// a step's first slice and A's in its second, so each slice issues half a
// step's loads.  When the rows' 128-byte K-segments cross cache lines, a
// step's load burst backs up between L1 and L2: at 8192^2 x 8200 the L1
// makes twice the L2 read requests it makes at 8192^3 and its
// TCP_TCR_TCP_STALL_CYCLES rise 9x, while the vendor library's kernel, with
// the same request counts, shows no such rise.  Halving the burst recovers
// most of the loss, and also helps a pitch of 129 lines.  Measured on MI355X
// (TFLOP/s, two stages / three B stages): 8192^2 x 8200 1215 / 1330,
// 8192^2 x 8136 1167 / 1278, 8192^2 x 8256 1431 / 1496, 4096^2 x 4104
// 1196 / 1307, 3000 x 5000 x 2056 1016 / 1127, 16384^2 x 1032 991 / 1079;
// with K % 512 == 0 the two are alike (8192^3 1505 / 1502, 4096^3 1412 /
// 1423, 3000 x 5000 x 2048 1195 / 1193, 16384^2 x 1024 1204 / 1189), and
// those keep the two-stage ring.
using BigDma3 = DmaCfg<256, 256, 2, 2, 64, 2, 16, 16, false, false, true>;
// 128 x 128: 4 waves of 64 x 64 on 16x16x32 MFMAs, four 32 KB stages.
using MidDma = DmaCfg<128, 128, 2, 2, 64, 4, 16, 16, true>;
// The same tile with two 32 KB stages: two workgroups share a CU, so one's
// prologue, epilogue and waits run under the other's MFMAs.  Measured on
// MI355X (TFLOP/s, two stages / four): 2048 x 4096 x 2048 (512 tiles)
// 1077 / 1033, 2304^2 x 4096 (324) 947 / 869, 1280 x 4096^2 (320) 943 / 866,
// 2560^2 x 2048 (400) 904 / 869, 2048 x 3072 x 1024 (384) 843 / 784.  With at
// most 256 tiles each CU runs one workgroup, and two stages then hide too
// little load latency: 2048^3 (256) 705-734 / 905-1013, 1792^2 x 8192 (196)
// 711-769 / 1001-1079 (also with one workgroup per CU forced by padding the
// LDS request: 720 at 2048^3).  So it serves calls with more tiles than CUs.
using Mid2Dma = DmaCfg<128, 128, 2, 2, 64, 2, 16, 16, false>;
// 256 x 128: 4 waves of 128 x 64 (128 AGPRs each), three 48 KB stages, the
// refill split over two slices.  For shapes whose 128 x 128 tiles fill the
// CUs twice and whose 256 x 256 tiles leave CUs idle: one of these per CU
// does the same work as two 128 x 128 tiles with a quarter fewer loads and
// twice the MFMAs per barrier.  Measured (TFLOP/s, this / two 128 x 128 per
// CU): 8192x1024x4096 1185/1124, 4096x2048x4096 1180/1120, 1024x8192x8192
// 1248/1141; two stages instead of three: 4-10 % slower, 8 waves of 64 x 64:
// within 1 %.  Where the 256 x 256 tile fills the CUs it stays ahead
// (8192x2048x8192 1267 against 1424, 8192^3 1269 against 1429).
using RectDma = DmaCfg<256, 128, 2, 2, 64, 3, 16, 16, true>;
// 64 x 64 (skinny, HBM-bound shapes): 4 waves of 32 x 32 on 16x16x32 MFMAs,
// eight 16 KB stages so that each CU keeps ~112 KB of loads in flight.
using ThinDma = DmaCfg<64, 64, 2, 2, 64, 8, 16, 16, false>;
// 64 x 32 and 32 x 64 (skinny shapes whose 64 x 64 tiles would leave CUs
// idle, e.g. 64 x 8192 x K): 2 waves of 32 x 32, ten 12 KB stages.
using ThinNDma = DmaCfg<64, 32, 2, 1, 64, 10, 16, 16, false>;
using ThinMDma = DmaCfg<32, 64, 1, 2, 64, 10, 16, 16, false>;
// 4-byte loads (FP8 with K % 4 == 0, operands 4-byte aligned): four times
// as many load instructions per step, so fewer stages keep the waits
// encodable.
using ThinDma4 = DmaCfg<64, 64, 2, 2, 64, 4, 16, 4, false>;
// Register-staged 16-byte chunks (any K, operands 2-byte aligned; taken for
// K < 8 and for skinny shapes whose rows are not 16-byte aligned, see
// load_bytes): two stages, each chunk loaded a step ahead into registers.
// The 256 x 256 tile
// runs 8 waves of 128 x 64 on 32x32x16 MFMAs, two per SIMD, each with its
// accumulators, fragments and 32 staging registers in 250 arch VGPRs: while
// one wave waits for a chunk the other multiplies.  Measured on MI355X
// (TFLOP/s, 8 waves / 4 waves of 128 x 128 with 64 staging registers):
// 3000 x 5000 x 2050 896 / 858, x 2049 871 / 833, 8192^2 x 8194 1170 / 1162,
// 4096^2 x 4097 1037 / 1025, when those shapes still ran here.  (4 waves
// with 16x16x32 blocks spill.)
using BigReg = DmaCfg<256, 256, 2, 4, 64, 2, 32, 16, false, true>;
using MidReg = DmaCfg<128, 128, 2, 2, 64, 2, 16, 16, false, true>;
using ThinReg = DmaCfg<64, 64, 2, 2, 64, 2, 16, 16, false, true>;

enum class Tile { kBig, kMid, kThin, kThinN, kThinM, kRect };

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile choice: the one with the smaller (waves of workgroups) x (time of one
// tile), one workgroup per CU on MI355X's 256 CUs.  Tile times relative to a
// 128 x 128 x K tile at the big tile's rate, measured on MI355X: a 256 x 256
// tile costs 4.0, a 128 x 128 tile 1.4 and a 64 x 64 tile 0.85 with 16-byte
// loads (the big tile's pipeline is ~40 % faster per FLOP; the 64 x 64 tile
// moves more bytes per FLOP but fills four times as many CUs); with 4-byte
// loads (K % 8 != 0) 6.6, 2.25 and 1.3.  So 3000 x 5000 runs one wave of 240
// big tiles rather than four of 960 mid tiles, 2048 x 2048 runs 256 mid tiles
// rather than 64 big ones, and 1024 x 1024 runs 256 thin tiles rather than
// 64 mid ones (5.5 against 8.1 us at K = 1024).  The choice assumes operands
// aligned to 16 bytes.
constexpr int kCUs = 256;

// thin_ok = false (FP8, whose 64 x 64 tile cost is not measured): the thin
// tile only when M or N is at most 64.
inline Tile choose_tile(int64_t M, int64_t N, int64_t K, bool thin_ok = true)
{
    if (M <= 64 || N <= 64) {
        // Skinny: every CU streams its share of the long operand, so fewer
        // than one 64 x 64 tile per CU leaves bandwidth unused; halving the
        // tile along the long side then fills twice as many CUs.
        if (thin_ok && cdiv(M, 64) * cdiv(N, 64) < kCUs) {
            if (M <= 64 && N > 64)
                return Tile::kThinN;
            if (N <= 64 && M > 64)
                return Tile::kThinM;
        }
        return Tile::kThin;
    }
    const bool wide = K >= 8;      // 16-byte direct-to-LDS loads (load_bytes, M, N > 64)
    const double big_tile = wide ? 4.0 : 6.6, mid_tile = wide ? 1.4 : 2.25;
    const double thin_tile = wide ? 0.85 : 1.3, rect_tile = 2.67;
    const double big = cdiv(cdiv(M, 256) * cdiv(N, 256), kCUs) * big_tile;
    const double mid = cdiv(cdiv(M, 128) * cdiv(N, 128), kCUs) * mid_tile;
    const double thin = cdiv(cdiv(M, 64) * cdiv(N, 64), kCUs) * thin_tile;
    if (!thin_ok)
        return big <= mid ? Tile::kBig : Tile::kMid;
    // the 256 x 128 tile only on direct loads (register staging would run
    // the 128 x 128 kernel) and with K >= 1024: below that, two 128 x 128
    // workgroups per CU hide each other's prologue and epilogue (TFLOP/s,
    // 256 x 128 / two-stage 128 x 128: 4096x2048x256 447/484, x512 729/744,
    // 8192x1024x1024 1012/978, 2560^2x2048 1019/969, 2560^2x2050 792/671)
    const double rect = wide && K >= 1024
                            ? cdiv(cdiv(M, 256) * cdiv(N, 128), kCUs) * rect_tile
                            : 1e30;
    if (big <= mid && big <= thin && big <= rect)
        return Tile::kBig;
    if (rect < mid && rect <= thin)
        return Tile::kRect;
    return mid <= thin ? Tile::kMid : Tile::kThin;
}

// The tile a call runs: register staging (direct == false) serves the
// 64 x 32 and 32 x 64 tiles with the 64 x 64 kernel and the 256 x 128 tile
// with the 128 x 128 one.
inline Tile run_tile(Tile t, bool direct)
{
    if (!direct && t == Tile::kRect)
        return Tile::kMid;
    return !direct && (t == Tile::kThinN || t == Tile::kThinM) ? Tile::kThin : t;
}

inline void tile_dims(Tile t, int &bm, int &bn)
{
    switch (t) {
    case Tile::kBig: bm = BigDma::BM; bn = BigDma::BN; break;
    case Tile::kMid: bm = MidDma::BM; bn = MidDma::BN; break;
    case Tile::kRect: bm = RectDma::BM; bn = RectDma::BN; break;
    case Tile::kThinN: bm = ThinNDma::BM; bn = ThinNDma::BN; break;
    case Tile::kThinM: bm = ThinMDma::BM; bn = ThinMDma::BN; break;
    default: bm = ThinDma::BM; bn = ThinDma::BN; break;
    }
}

// Sizes every entry point accepts: M, N in [0, 2^31 - 1], K in [0, GEMM_MAX_K].
inline bool sizes_ok(int64_t M, int64_t N, int64_t K)
{
    return M >= 0 && N >= 0 && K >= 0 && M <= INT32_MAX && N <= INT32_MAX && K <= GEMM_MAX_K;
}

inline int validate(const void *A, const void *B, const void *D, int64_t M, int64_t N, int64_t K)
{
    if (!sizes_ok(M, N, K))
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

template <bool EPI>
EpiArg<EPI> epi_arg(const Epi &e)
{
    if constexpr (EPI)
        return e;
    else
        return NoEpi{};
}

// Grid of a one-tile-per-workgroup launch: at least `tiles` workgroups.  A
// grid dimension holds at most 2^32 - 1 work-items, so tile counts above
// 2^22 (workgroups of up to 512 lanes) spread over y; the kernel numbers its
// tile blockIdx.x + blockIdx.y * gridDim.x and skips those past the last.
inline dim3 tile_grid(int64_t tiles)
{
    constexpr int64_t kMaxX = int64_t(1) << 22;
    if (tiles <= kMaxX)
        return dim3((unsigned)tiles);
    return dim3((unsigned)kMaxX, (unsigned)cdiv(tiles, kMaxX));
}

template <class C, bool SK, bool EPI, bool BF>
void launch_dma(const void *A, const void *B, void *D, int M, int N, int K, int vec, hipStream_t s,
                const SkPlan &sk, int grid, const Epi &epi)
{
    using T = typename Elem<BF>::T;
    const int tm = (int)cdiv(M, C::BM), tn = (int)cdiv(N, C::BN);
    const dim3 g = SK ? dim3((unsigned)grid) : tile_grid((int64_t)tm * tn);
    auto go = [&](auto ktail, auto ntc) {
        hipLaunchKernelGGL((gemm_nt_dma_kernel<C, decltype(ktail)::value, SK, EPI, BF, 0, 2,
                                               decltype(ntc)::value>),
                           g, dim3(C::THREADS), 0, s, (const T *)A,
                           (const T *)B, (T *)D, M, N, K, tm, tn, vec, sk, epi_arg<EPI>(epi));
    };
    auto go_nt = [&](auto ktail) {
        // An operand read once per call (one tile row: B; one tile column:
        // A) streams with the non-temporal policy: 64 x 16384 x 8192 with
        // operands streamed from HBM reads 5.26 TB/s instead of 4.66 (but
        // 5.36 instead of 6.0 when B stays resident in the last-level cache
        // between calls).  The 128 x 128 and 64 x 64 direct-load tiles only.
        const int nt = (C::BM <= 128 && !C::REG && !SK) ? (tn == 1 ? 1 : 0) | (tm == 1 ? 2 : 0) : 0;
        if constexpr (C::BM <= 128 && !C::REG && !SK) {
            switch (nt) {
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

// The kernels' vec_store flag: 0 element stores; 1 D (and the epilogue's C
// and bias, `other`) 8-byte aligned and N % 4 == 0: 8-byte stores and loads;
// 2 also D 16-byte aligned and N % 8 == 0: whole tiles go through the LDS
// staged epilogue (the direct-to-LDS kernels with 16x16 blocks).
inline int store_mode(const void *D, int64_t N, uintptr_t other = 0)
{
    const uintptr_t d = (uintptr_t)D;
    if (((d | other) & 7u) != 0 || N % 4 != 0)
        return 0;
    return ((d & 15u) == 0 && N % 8 == 0) ? 2 : 1;
}

// Bytes each lane moves per direct-to-LDS load for these operands: 16, or 0
// for the register-staged kernel.  Rows that start 16-byte aligned (K % 8
// == 0, A and B 16-byte aligned) always take the direct loads.  The 16-byte
// direct-to-LDS loads also take any 2-byte aligned address on gfx950, so
// rows that do not (K % 8 != 0, or operands offset by whole elements) take
// them too, with two exceptions that stay with register staging: K < 8
// (the first K-step's fix-up reads 16 bytes from each row's start, which a
// row of fewer than 8 elements does not span) and skinny shapes (M or N <=
// 64), whose tiles stream the long operand from HBM faster with register
// staging at such rows (measured on MI355X, TFLOP/s, direct / register-
// staged: 64 x 32768 x 4095 182 / 240, 64 x 16384 x 8191 224 / 249;
// elsewhere direct wins: 3000 x 5000 x 2050 1023-1080 / 847, 8192^2 x 8191
// 1174 / 1046, 2048^2 x 2047 648-668 / 591, 1024^2 x 4095 367 / 337).
inline int load_bytes(const void *A, const void *B, int64_t M, int64_t N, int64_t K)
{
    const uintptr_t ab = (uintptr_t)A | (uintptr_t)B;
    if (K % 8 == 0 && (ab & 15u) == 0)
        return 16;
    return K >= 8 && (ab & 1u) == 0 && M > 64 && N > 64 ? 16 : 0;
}

// One workgroup per tile.  EPI: with the fused epilogue `epi`, whose C and
// bias must then also be 8-byte aligned for vector accesses.  CDma: the
// direct-to-LDS pipeline (K % 8 == 0, A and B 16-byte aligned); CReg: the
// same pipeline with register-staged 16-byte chunks (everything else).
template <class CDma, class CReg, bool EPI = false, bool BF = false>
void launch_tile(const void *A, const void *B, void *D, int M, int N, int K, hipStream_t s,
                 const Epi &epi = Epi{})
{
    const int vec = store_mode(D, N, (uintptr_t)epi.C | (uintptr_t)epi.bias);
    const SkPlan none{};
    if (load_bytes(A, B, M, N, K) == 16)
        launch_dma<CDma, false, EPI, BF>(A, B, D, M, N, K, vec, s, none, 0, epi);
    else
        launch_dma<CReg, false, EPI, BF>(A, B, D, M, N, K, vec, s, none, 0, epi);
}

// The tile `t` with direct-to-LDS loads when they apply, else register
// staging (the 64 x 64 kernel serves the 64 x 32 and 32 x 64 tiles then).
template <bool EPI = false, bool BF = false>
void launch_plain(Tile t, const void *A, const void *B, void *D, int M, int N, int K,
                  hipStream_t s, const Epi &epi = Epi{})
{
    switch (t) {
    case Tile::kBig:
        if (K % 512 != 0)
            launch_tile<BigDma3, BigReg, EPI, BF>(A, B, D, M, N, K, s, epi);
        else
            launch_tile<BigDma, BigReg, EPI, BF>(A, B, D, M, N, K, s, epi);
        break;
    case Tile::kMid:
        if (cdiv(M, 128) * cdiv(N, 128) > kCUs)
            launch_tile<Mid2Dma, MidReg, EPI, BF>(A, B, D, M, N, K, s, epi);
        else
            launch_tile<MidDma, MidReg, EPI, BF>(A, B, D, M, N, K, s, epi);
        break;
    case Tile::kRect: launch_tile<RectDma, MidReg, EPI, BF>(A, B, D, M, N, K, s, epi); break;
    case Tile::kThinN: launch_tile<ThinNDma, ThinReg, EPI, BF>(A, B, D, M, N, K, s, epi); break;
    case Tile::kThinM: launch_tile<ThinMDma, ThinReg, EPI, BF>(A, B, D, M, N, K, s, epi); break;
    default: launch_tile<ThinDma, ThinReg, EPI, BF>(A, B, D, M, N, K, s, epi); break;
    }
}

// ---------------------------------------------------------------------------
// Stream-K planning.  Measured on MI355X (TFLOPS, stream-K / 128 x 128 tiles
// / 64 x 64 tiles, one workgroup per tile): 1024^2x16384 833/433/740,
// 512x640x16384 307/136/273, 1024^2x8192 613/407/676, 768x1024x8192
// 494/314/559, 1024^2x4100 322/220/379; and earlier 1280^2x8192 444/624,
// 1536^2x8192 684/792 (stream-K / 128 x 128).  Stream-K runs on the 128 x 128
// tile when those tiles fill at most a quarter of the CUs and K spans at
// least 192 K-steps: the partial-sum hand-off (one fp32 tile per contributor
// through memory) then costs less than the 64 x 64 tiles' extra loads, which
// win below that.  The 256 x 256 tile is not used for it: its hand-off moves
// 256 KB per contributor and its pipeline leaves no registers for the
// persistent loop.
struct Plan {
    Tile tile = Tile::kThin;
    bool sk = false;
    int grid = 0;
    SkPlan split{};
};

// Stream-K split of `tiles` tiles of `steps` K-steps over P workgroups: if
// there are fewer tiles than workgroups, every tile; otherwise the last
// partial wave plus one full wave is split by steps (each workgroup then
// gets between one and two tiles of work) and the rest run whole.
inline SkPlan sk_split(int64_t tiles, int64_t steps, int P)
{
    SkPlan sp{};
    sp.sk_tiles = (int)(tiles < P ? tiles : tiles % P + P);
    sp.dp_tiles = (int)(tiles - sp.sk_tiles);
    const int64_t total = (int64_t)sp.sk_tiles * steps;
    sp.base = (int)(total / P);
    sp.extra = (int)(total % P);
    return sp;
}

constexpr int64_t kSkMinSteps = 192;

// Skinny shapes (M or N <= 64; 16-byte loads, so K % 8 == 0): the plain grid
// runs one 64 x 32 (or 32 x 64) tile per workgroup, which leaves CUs idle
// when there are fewer tiles than CUs, and every tile re-reads the whole
// short operand.  Stream-K then runs on the 64 x 64 tile (half the re-reads)
// when there are P/4 to P/2 of those tiles and either CUs idle or the K-loop
// is long (>= 128 steps), else on the plain tile when it fills at most half
// the CUs and every workgroup gets >= 8 K-steps.  Measured on MI355X, kernel
// us, plain / stream-K on 64 x 32 / stream-K on 64 x 64: 64x2048x8192
// 24.0/13.2/12.8, 64x1024x8192 26.1/13.9/16.3, 64x512x8192 25.9/16.8/25.6,
// 64x256x16384 48.7/24.9/42.0, 64x2048x4096 14.7/11.1/12.7, 64x4096x4096
// 15.1/12.3/10.9, 64x6144x8192 29.7/22.5/21.5, 64x8192x8192 31.4/26.2/25.2,
// 8192x64x8192 30.9/26.3/25.5, 32x8192x4096 14.3/16.1/16.4; fewer K-steps or
// per-workgroup steps lose to the plain grid (64x2048x2048 8.8/10.1,
// 64x512x4096 13.9/16.4, one 64 x 64 tile at K = 8192 36/75).
inline bool plan_skinny(Plan &pl, int64_t M, int64_t N, int64_t K, int P)
{
    const int64_t steps = cdiv(K, 64);
    if (K % 8 != 0 || steps < 64)
        return false;
    int bm, bn;
    tile_dims(pl.tile, bm, bn);
    const int64_t plain = cdiv(M, bm) * cdiv(N, bn);
    const int64_t t64 = cdiv(M, 64) * cdiv(N, 64);
    int64_t tiles;
    if (4 * t64 >= P && 2 * t64 <= P && (plain < P || steps >= 128)) {
        pl.tile = Tile::kThin;
        tiles = t64;
    } else if (2 * plain <= P && plain * steps >= 8 * (int64_t)P) {
        tiles = plain;
    } else {
        return false;
    }
    pl.sk = true;
    pl.grid = P;
    pl.split = sk_split(tiles, steps, P);
    return true;
}

// lb: 16 (0: the register-staged path, no stream-K).
inline Plan make_plan(int64_t M, int64_t N, int64_t K, int lb, int P)
{
    Plan pl;
    pl.tile = choose_tile(M, N, K);
    if (lb == 0 || K == 0)
        return pl;
    if (M <= 64 || N <= 64) {
        plan_skinny(pl, M, N, K, P);
        return pl;
    }
    const int64_t steps = cdiv(K, 64);
    const int64_t tiles = cdiv(M, 128) * cdiv(N, 128);
    if (4 * tiles <= P && steps >= kSkMinSteps) {
        pl.tile = Tile::kMid;
        pl.sk = true;
        pl.grid = P;
        pl.split = sk_split(tiles, steps, P);
    }
    return pl;
}

inline int64_t flag_bytes(int P) { return cdiv((int64_t)P * 4, 256) * 256; }
constexpr int64_t kSkHdrBytes = kSkHdrWords * 4;

inline int64_t workspace_bytes(const Plan &pl)
{
    if (!pl.sk)
        return 0;
    int bm, bn;
    tile_dims(pl.tile, bm, bn);
    return kSkHdrBytes + flag_bytes(pl.grid) + (int64_t)pl.grid * bm * bn * 4;
}

// The persistent stream-K grid on the plan's tile (direct-to-LDS paths).
inline void launch_sk(const void *A, const void *B, void *D, int M, int N, int K, hipStream_t s,
                      const SkPlan &sk, int grid, Tile t)
{
    const int vec = (((uintptr_t)D & 7u) == 0 && N % 4 == 0) ? 1 : 0;
    switch (t) {
    case Tile::kThin:
        launch_dma<ThinDma, true, false, false>(A, B, D, M, N, K, vec, s, sk, grid, Epi{});
        break;
    case Tile::kThinN:
        launch_dma<ThinNDma, true, false, false>(A, B, D, M, N, K, vec, s, sk, grid, Epi{});
        break;
    case Tile::kThinM:
        launch_dma<ThinMDma, true, false, false>(A, B, D, M, N, K, vec, s, sk, grid, Epi{});
        break;
    default:
        launch_dma<MidDma, true, false, false>(A, B, D, M, N, K, vec, s, sk, grid, Epi{});
        break;
    }
}

// Header, flags and slots of a stream-K plan inside workspace `ws`.
inline void bind_workspace(SkPlan &sp, void *ws, int grid)
{
    sp.hdr = (uint32_t *)ws;
    sp.flags = (uint32_t *)((char *)ws + kSkHdrBytes);
    sp.partials = (float *)((char *)ws + kSkHdrBytes + flag_bytes(grid));
}

// Workgroups the stream-K grid may use on the current device: one per CU,
// at most kCUs.  The count is read once per device.
inline int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return kCUs;
    if (dev >= 0 && dev < 64 && (cus = cache[dev].load(std::memory_order_relaxed)) > 0)
        return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return kCUs;
    cus = cus < kCUs ? cus : kCUs;
    if (dev >= 0 && dev < 64)
        cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

} // namespace
