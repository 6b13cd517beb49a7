/*
 * gemm_nt_f16.h -- C ABI of the dense fp16 "NT" GEMM for AMD MI355X (gfx950).
 *
 * Operation (page "构建 Tiled GEMM" / "Building a Tiled GEMM", mlc.ai
 * modern-gpu-programming-for-mlsys, chapter gemm_basics, section "GEMM"):
 *
 *     D[m,n] = sum_{k<K} A[m,k] * B[n,k]       0 <= m < M, 0 <= n < N
 *
 * A is M x K, B is N x K (the linear-layer weight layout, so D = A * B^T
 * with no transpose or reordering of B), D is M x N.  A, B and D are stored
 * as IEEE binary16 (fp16); products are accumulated in fp32 and the sum is
 * converted to fp16 with round-to-nearest-even.  The same page defines the
 * throughput measure TFLOPS = 2*M*N*K / (t * 1e12).
 *
 * Layout: every matrix is dense row-major with no padding: element (r, c) of
 * A is at A[r*K + c], of B at B[r*K + c], of D at D[r*N + c].
 *
 * Ownership: the caller allocates A, B and D in device memory (any 2-byte
 * aligned address) and keeps them alive until the work enqueued on `stream`
 * has finished.  The library allocates no device memory, keeps no pointer
 * after a call returns, writes every element of D and nothing outside
 * [D, D + M*N).
 *
 * Streams: work is enqueued on `stream` (NULL = the null stream) and the call
 * returns without waiting for it.  Faults inside a kernel are not reported by
 * the return code; the caller sees them at its next synchronisation.
 *
 * Errors: every argument check happens before any HIP runtime call, so the
 * checks can be exercised on a machine without a GPU.
 *
 * Thread safety: every entry point is re-entrant; the library holds no
 * mutable state.
 */
#ifndef GEMM_NT_F16_H
#define GEMM_NT_F16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as the HIP runtime's stream handle. */
typedef struct ihipStream_t *hipStream_t;

/* Return codes. */
#define GEMM_OK 0       /* work enqueued (or nothing to do)                    */
#define GEMM_EINVAL 1   /* argument rejected; nothing enqueued                 */
#define GEMM_ELAUNCH 2  /* the HIP runtime reported an error at kernel launch  */

/* Largest K accepted: a 256-row operand panel must span fewer than 2^31
 * bytes, the range one buffer resource addresses. */
#define GEMM_MAX_K 4194303

/*
 * D = A * B^T in fp16 with fp32 accumulation (the operation above).
 *
 * A: M x K fp16, B: N x K fp16, D: M x N fp16, all device pointers.
 * M, N, K: sizes, each in [0, 2^31 - 1]; K <= GEMM_MAX_K.
 * stream: HIP stream to enqueue on.
 *
 * Degenerate sizes: M == 0 or N == 0 enqueues nothing; K == 0 sets every
 * element of D to +0 (the empty sum).
 *
 * Returns GEMM_OK, GEMM_EINVAL (a size out of range, a NULL pointer for an
 * operand with at least one element, a pointer not 2-byte aligned, or D
 * overlapping A or B) or GEMM_ELAUNCH.
 */
int gemm_nt_f16(const void *A, const void *B, void *D,
                int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Static text for a return code; never NULL. */
const char *gemm_nt_f16_strerror(int code);

/*
 * Host-only introspection (no HIP call): the output tile BM x BN and the K
 * step BK that gemm_nt_f16 uses for an M x N x K problem with operands
 * aligned to 16 bytes, and the number of workgroups it launches.  Tests use
 * it to pick rows and columns at tile edges.  Returns GEMM_OK or GEMM_EINVAL
 * (negative size or NULL output).
 */
int gemm_nt_f16_tile(int64_t M, int64_t N, int64_t K,
                     int *bm, int *bn, int *bk, int64_t *workgroups);

/*
 * Host-only introspection (no HIP call): the output tile (tile_m, tile_n)
 * that workgroup `wg` computes when the output is split into tiles_m x
 * tiles_n tiles.  The map is a bijection of [0, tiles_m*tiles_n) onto the
 * tiles; it keeps tiles that share A or B rows on the same L2 slice.
 * Returns GEMM_OK or GEMM_EINVAL (wg or a count out of range, NULL output).
 */
int gemm_nt_f16_tile_coord(int64_t wg, int64_t tiles_m, int64_t tiles_n,
                           int64_t *tile_m, int64_t *tile_n);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_NT_F16_H */
