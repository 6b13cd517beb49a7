/*
 * gemm_oracle.c -- CPU oracle for the dense fp16 "NT" GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it: only the tests, the smoke
 * check and the benchmark's CPU-baseline leg use it.  It shares no code,
 * header or table with the HIP library.
 *
 * What it computes (page "构建 Tiled GEMM" / "Building a Tiled GEMM",
 * mlc.ai modern-gpu-programming-for-mlsys, chapter gemm_basics, section
 * "GEMM"):
 *
 *     D[m,n] = sum_{k<K} A[m,k] * B[n,k]
 *
 * A is M x K, B is stored N x K (the linear-layer weight layout; the product
 * equals A * B^T and B is never transposed), D is M x N.  All three are
 * dense row-major IEEE binary16 arrays.  The same page stores A, B and D in
 * fp16 and accumulates in a wider type; the oracle widens every fp16 input to
 * fp64 exactly, sums in fp64 in ascending k starting from +0.0, and rounds the
 * final sum once, directly from fp64 to fp16, round-to-nearest-ties-to-even.
 * The same index formula (row * K + k for the operands, row * N + col for
 * the output) is the one the naive kernel of page "如何用 Croqtile 一步步优化
 * 矩阵乘法内核" (section "内核 0：朴素版", Kernel 0: naive) evaluates.
 *
 * Readings taken where the pages are silent:
 *  - rounding of the final cast: IEEE round-to-nearest, ties-to-even;
 *  - magnitudes >= 65520 round to +-inf; subnormal fp16 inputs are honoured;
 *  - an exact-zero sum is +0 (the sum starts from +0.0);
 *  - K = 0 gives D = +0 everywhere (the empty sum);
 *  - NaN results are returned as the canonical quiet NaN 0x7E00.
 *
 * Fused epilogue (oracle_gemm_nt_f16_ex): the standard GEMM form that
 * scales the product and adds a scaled second matrix and a bias,
 *
 *     D[m,n] = alpha * sum_k A[m,k] * B[n,k] + beta * C[m,n] + bias[n]
 *
 * with C an M x N fp16 matrix and bias one fp16 value per output column (a
 * linear layer's bias).  Readings taken: alpha and beta are fp32 values
 * (widened exactly); the three terms are formed and added in fp64 in the
 * order written, and the result is rounded once to fp16; when beta == 0, C
 * is not read (BLAS convention) and contributes nothing; a missing bias is 0.
 *
 * bfloat16 (oracle_gemm_nt_bf16): the same definition on bfloat16 storage
 * (1 sign bit, 8 exponent bits with bias 127, 7 fraction bits: the upper
 * half of an IEEE binary32), decoded exactly, summed in fp64 and rounded
 * once to bfloat16 with round to nearest, ties to even.
 *
 * FP8 (oracle_gemm_nt_fp8): the GEMM-optimisation article at www.lqnn.cn
 * (news/123226) names the two 8-bit formats, E4M3 and E5M2 (section 2.2),
 * quantises with a scale kept in fp32 that maps the largest magnitude to
 * 448 (section 4.2) and undoes it in the kernel's epilogue.  Readings
 * taken: the formats are the OCP ones, E4M3 with bias 7, no infinities,
 * S.1111.111 the only NaN, largest finite 448 (the article's own 448; its
 * "range about 240" in section 2.2 does not fit that format), and E5M2 with
 * bias 15 and IEEE-style infinities and NaNs; each operand is decoded
 * exactly, the sum is taken in fp64, multiplied by one fp32 scale (the
 * product of A's and B's per-tensor dequantisation scales) and rounded once
 * to fp16.
 *
 * FP8 with per-channel weight scales (oracle_gemm_nt_fp8_cs): the same
 * article's weight quantisation (section 4.2, step 1) takes one scale per
 * output channel, the largest magnitude of each weight row over 448, and the
 * activation one scale per tensor from calibration (step 2).  In this layout
 * a weight row is a row n of B, so column n of D takes the scale
 * s_n = a_scale * b_scale[n].  Reading taken: s_n is formed in fp32 (one
 * rounding, as both scales are fp32 values), then multiplies the exact sum
 * before the one rounding to fp16.
 *
 * fp16 accumulation (oracle_gemm_nt_f16_acc16): page "如何用 Croqtile 一步步
 * 优化矩阵乘法内核" keeps the running sum itself in fp16: its naive kernel
 * declares an f16 accumulator (section "内核 0：朴素版"), and its Hopper
 * kernels fill the matrix-unit accumulator as f16, which it notes takes
 * fewer registers (section "内核 2：Hopper TMA + WGMMA"; the tuned kernel of
 * section "内核 4：生产级调优" keeps it): the running sum is an fp16 value and
 * every update of it is an fp16 addition.  Readings taken where the page is
 * silent:
 *  - one update adds the products of 64 consecutive k (a chunk); the chunks
 *    tile [0, K) from its end, so when K is not a multiple of 64 the first
 *    chunk holds the K mod 64 leading terms;
 *  - the chunk's products are summed (in fp64) and the sum rounded to fp16,
 *    then added to s with an fp16 addition: s <- fp16(s + fp16(chunk sum)),
 *    each rounding to nearest with ties to even;
 *  - s starts at +0 and D[m,n] is the last s; K = 0 gives +0; an infinite
 *    or NaN s stays so (NaN as 0x7E00).  A chunk sum that rounds to -0
 *    adds as +0 + -0 = +0, so D is never -0.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no -ffast-math:
 * the sum must be evaluated exactly in the written order).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- binary16 decode, from the IEEE 754 binary16 definition ------------
 * Layout: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-24
 *   exponent 1..30  : normal,    value = (1024 + fraction) * 2^(exponent-25)
 *   exponent 31     : infinity (fraction 0) or NaN (fraction != 0)        */
static double f16_decode(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/* ---- fp64 -> binary16, round to nearest, ties to even ------------------
 * Take |x| in binade [2^E, 2^(E+1)).  Normal fp16 numbers in that binade are
 * integer multiples of the quantum 2^(E-10); below 2^-14 the quantum is fixed
 * at 2^-24 (subnormals).  Scale |x| by the inverse quantum (a power of two,
 * so exact), round the scaled value to an integer with ties to even, then
 * re-assemble.  A carry to 2048 moves to the next binade; a binade above 15
 * is infinity.                                                            */
static uint16_t f16_encode_rne(double x)
{
    if (isnan(x))
        return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    int e2;
    (void)frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1)     */
    int E = e2 - 1;               /* a in [2^E, 2^(E+1))               */
    if (E > 15)
        return sign | 0x7c00;     /* >= 65536: beyond every rounding   */
    if (E < -14)
        E = -14;                  /* subnormal quantum 2^-24           */
    double scaled = ldexp(a, 10 - E);   /* exact power-of-two scaling  */
    double lo = floor(scaled);
    double rem = scaled - lo;           /* exact: scaled < 2^11        */
    long n = (long)lo;
    if (rem > 0.5 || (rem == 0.5 && (n & 1)))
        n += 1;
    if (n == 2048) {              /* rounded up into the next binade   */
        n = 1024;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c00;
    if (n < 1024)                 /* only possible when E == -14       */
        return sign | (uint16_t)n;
    return sign | (uint16_t)(((E + 15) << 10) | (n - 1024));
}

/* ---- bfloat16 decode and encode ----------------------------------------
 * Layout: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 *   exponent 0       : subnormal, value = fraction * 2^-133
 *   exponent 1..254  : normal,    value = (128 + fraction) * 2^(exponent-134)
 *   exponent 255     : infinity (fraction 0) or NaN                      */
static double bf16_decode(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 7) & 0xff;
    int frac = h & 0x7f;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -133);
    else if (expo == 255)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + frac), expo - 134);
    return sign ? -v : v;
}

/* fp64 -> bfloat16, round to nearest, ties to even: the same construction as
 * f16_encode_rne with 7 fraction bits, minimum normal exponent -126 and
 * maximum 127.                                                            */
static uint16_t bf16_encode_rne(double x)
{
    if (isnan(x))
        return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7f80;
    if (a == 0.0)
        return sign;
    int e2;
    (void)frexp(a, &e2);
    int E = e2 - 1;               /* a in [2^E, 2^(E+1))               */
    if (E > 127)
        return sign | 0x7f80;
    if (E < -126)
        E = -126;                 /* subnormal quantum 2^-133          */
    double scaled = ldexp(a, 7 - E);
    double lo = floor(scaled);
    double rem = scaled - lo;
    long n = (long)lo;
    if (rem > 0.5 || (rem == 0.5 && (n & 1)))
        n += 1;
    if (n == 256) {
        n = 128;
        E += 1;
    }
    if (E > 127)
        return sign | 0x7f80;
    if (n < 128)
        return sign | (uint16_t)n;
    return sign | (uint16_t)(((E + 127) << 7) | (n - 128));
}

static double g_lut_bf[65536];
static int g_lut_bf_ready = 0;

static void lut_bf_init(void)
{
    if (g_lut_bf_ready)
        return;
    for (int h = 0; h < 65536; ++h)
        g_lut_bf[h] = bf16_decode((uint16_t)h);
    g_lut_bf_ready = 1;
}

/* Decoded value of every binary16 pattern, filled once from f16_decode. */
static double g_lut[65536];
static int g_lut_ready = 0;

static void lut_init(void)
{
    if (g_lut_ready)
        return;
    for (int h = 0; h < 65536; ++h)
        g_lut[h] = f16_decode((uint16_t)h);
    g_lut_ready = 1;
}

static int pick_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* The fp64 sum of one output entry, ascending k from +0.0. */
static double dot(const uint16_t *arow, const uint16_t *brow, int64_t K)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += g_lut[arow[k]] * g_lut[brow[k]];
    return acc;
}

/* One output entry: the sum, rounded once. */
static uint16_t entry(const uint16_t *arow, const uint16_t *brow, int64_t K)
{
    return f16_encode_rne(dot(arow, brow, K));
}

/* ---- exported API ------------------------------------------------------ */

void oracle_f16_decode(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f16_decode(in[i]);
}

void oracle_f16_encode(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f16_encode_rne(in[i]);
}

/* Full D = A * B^T.  Rows of D are spread over threads; every entry's sum is
 * sequential.  Returns the number of threads used. */
int oracle_gemm_nt_f16(const uint16_t *A, const uint16_t *B, uint16_t *D,
                       int64_t M, int64_t N, int64_t K, int nthreads)
{
    lut_init();
    int nt = pick_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            D[m * N + n] = entry(A + m * K, B + n * K, K);
    return nt;
}

/* Selected entries D[rows[i], cols[i]], i < count.  Indices must lie in
 * [0, M) x [0, N); entries with an index outside get 0x7E00 (NaN) so that a
 * caller's mistake cannot pass silently.  Returns the number of threads. */
int oracle_gemm_nt_f16_entries(const uint16_t *A, const uint16_t *B,
                               int64_t M, int64_t N, int64_t K,
                               const int64_t *rows, const int64_t *cols,
                               int64_t count, uint16_t *out, int nthreads)
{
    lut_init();
    int nt = pick_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = rows[i], n = cols[i];
        if (m < 0 || m >= M || n < 0 || n >= N)
            out[i] = 0x7e00;
        else
            out[i] = entry(A + m * K, B + n * K, K);
    }
    return nt;
}

/* Full D = alpha * (A * B^T) + beta * C + bias (see the header comment).
 * C may be NULL when beta == 0 (it is not read then); bias may be NULL. */
int oracle_gemm_nt_f16_ex(const uint16_t *A, const uint16_t *B, const uint16_t *C,
                          const uint16_t *bias, uint16_t *D, int64_t M, int64_t N, int64_t K,
                          float alpha, float beta, int nthreads)
{
    lut_init();
    int nt = pick_threads(nthreads);
    const double a = (double)alpha, b = (double)beta;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double r = a * dot(A + m * K, B + n * K, K);
            if (b != 0.0)
                r = r + b * g_lut[C[m * N + n]];
            if (bias)
                r = r + g_lut[bias[n]];
            D[m * N + n] = f16_encode_rne(r);
        }
    return nt;
}

/* ---- fp16 accumulation -------------------------------------------------- */

/* One output entry with an fp16 running sum: chunks of 64 consecutive k,
 * aligned to K's end; each chunk's sum, rounded to fp16, is added to the sum
 * with an fp16 addition (the exact sum of two fp16 values, rounded once). */
static uint16_t entry_acc16(const uint16_t *arow, const uint16_t *brow, int64_t K)
{
    double s = 0.0;                       /* always an fp16 value */
    int64_t k0 = 0;
    int64_t len = K % 64 ? K % 64 : 64;   /* the first chunk */
    while (k0 < K) {
        double c = 0.0;
        for (int64_t k = k0; k < k0 + len; ++k)
            c += g_lut[arow[k]] * g_lut[brow[k]];
        s = g_lut[f16_encode_rne(s + g_lut[f16_encode_rne(c)])];
        k0 += len;
        len = 64;
    }
    return f16_encode_rne(s);
}

/* Full D with an fp16 running sum (see the header comment). */
int oracle_gemm_nt_f16_acc16(const uint16_t *A, const uint16_t *B, uint16_t *D,
                             int64_t M, int64_t N, int64_t K, int nthreads)
{
    lut_init();
    int nt = pick_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            D[m * N + n] = entry_acc16(A + m * K, B + n * K, K);
    return nt;
}

/* Selected entries of the fp16-accumulated product (index outside: NaN). */
int oracle_gemm_nt_f16_acc16_entries(const uint16_t *A, const uint16_t *B,
                                     int64_t M, int64_t N, int64_t K,
                                     const int64_t *rows, const int64_t *cols,
                                     int64_t count, uint16_t *out, int nthreads)
{
    lut_init();
    int nt = pick_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = rows[i], n = cols[i];
        if (m < 0 || m >= M || n < 0 || n >= N)
            out[i] = 0x7e00;
        else
            out[i] = entry_acc16(A + m * K, B + n * K, K);
    }
    return nt;
}

/* ---- bfloat16 ---------------------------------------------------------- */

void oracle_bf16_decode(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_decode(in[i]);
}

void oracle_bf16_encode(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_encode_rne(in[i]);
}

static uint16_t entry_bf(const uint16_t *arow, const uint16_t *brow, int64_t K)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += g_lut_bf[arow[k]] * g_lut_bf[brow[k]];
    return bf16_encode_rne(acc);
}

/* Full D = A * B^T on bfloat16 storage. */
int oracle_gemm_nt_bf16(const uint16_t *A, const uint16_t *B, uint16_t *D,
                        int64_t M, int64_t N, int64_t K, int nthreads)
{
    lut_bf_init();
    int nt = pick_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            D[m * N + n] = entry_bf(A + m * K, B + n * K, K);
    return nt;
}

/* Selected entries of the bfloat16 product (index outside: 0x7FC0, NaN). */
int oracle_gemm_nt_bf16_entries(const uint16_t *A, const uint16_t *B,
                                int64_t M, int64_t N, int64_t K,
                                const int64_t *rows, const int64_t *cols,
                                int64_t count, uint16_t *out, int nthreads)
{
    lut_bf_init();
    int nt = pick_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = rows[i], n = cols[i];
        if (m < 0 || m >= M || n < 0 || n >= N)
            out[i] = 0x7fc0;
        else
            out[i] = entry_bf(A + m * K, B + n * K, K);
    }
    return nt;
}

/* ---- FP8 (OCP E4M3 and E5M2) --------------------------------------------
 * E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits; exponent 0 is
 * subnormal (fraction * 2^-9); S.1111.111 is NaN; no infinity.
 * E5M2: 1 sign, 5 exponent (bias 15), 2 fraction bits; exponent 0 is
 * subnormal (fraction * 2^-16); exponent 31 is infinity or NaN.           */
static double fp8_decode(uint8_t v, int e5m2)
{
    int sign = v >> 7;
    double x;
    if (!e5m2) {
        int e = (v >> 3) & 15, f = v & 7;
        if (e == 15 && f == 7)
            return NAN;
        x = e ? ldexp((double)(8 + f), e - 10) : ldexp((double)f, -9);
    } else {
        int e = (v >> 2) & 31, f = v & 3;
        if (e == 31)
            return f ? NAN : (sign ? -INFINITY : INFINITY);
        x = e ? ldexp((double)(4 + f), e - 17) : ldexp((double)f, -16);
    }
    return sign ? -x : x;
}

void oracle_fp8_decode(const uint8_t *in, double *out, int64_t n, int e5m2)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = fp8_decode(in[i], e5m2);
}

/* Full D = scale * (A * B^T) with A, B in FP8 (a_e5m2 / b_e5m2 select E5M2
 * over E4M3) and D in fp16. */
int oracle_gemm_nt_fp8(const uint8_t *A, const uint8_t *B, uint16_t *D, int64_t M, int64_t N,
                       int64_t K, int a_e5m2, int b_e5m2, float scale, int nthreads)
{
    double la[256], lb[256];
    for (int v = 0; v < 256; ++v) {
        la[v] = fp8_decode((uint8_t)v, a_e5m2);
        lb[v] = fp8_decode((uint8_t)v, b_e5m2);
    }
    int nt = pick_threads(nthreads);
    const double sc = (double)scale;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *ar = A + m * K, *br = B + n * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += la[ar[k]] * lb[br[k]];
            D[m * N + n] = f16_encode_rne(sc * acc);
        }
    return nt;
}

/* Per-channel form: D[m][n] = s_n * (A * B^T)[m][n] with s_n the fp32
 * product a_scale * b_scale[n] (b_scale: N values, one per row of B). */
int oracle_gemm_nt_fp8_cs(const uint8_t *A, const uint8_t *B, uint16_t *D, int64_t M, int64_t N,
                          int64_t K, int a_e5m2, int b_e5m2, float a_scale,
                          const float *b_scale, int nthreads)
{
    double la[256], lb[256];
    for (int v = 0; v < 256; ++v) {
        la[v] = fp8_decode((uint8_t)v, a_e5m2);
        lb[v] = fp8_decode((uint8_t)v, b_e5m2);
    }
    int nt = pick_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *ar = A + m * K, *br = B + n * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += la[ar[k]] * lb[br[k]];
            const float sn = a_scale * b_scale[n];
            D[m * N + n] = f16_encode_rne((double)sn * acc);
        }
    return nt;
}
