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
 * Thread safety: every entry point is re-entrant.  The library's only
 * mutable state is a per-device cache of the CU count (written once, with
 * atomic accesses) and the static workspace of gemm_nt_f16_ws_noalloc, whose
 * own comment states how calls share it.
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
#define GEMM_ESCRATCH 3 /* the call needs more than the library's static scratch */

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

/*
 * The same operation on bfloat16 storage: A, B and D hold bfloat16 (1 sign,
 * 8 exponent, 7 fraction bits), products are accumulated in fp32 and the sum
 * is converted to bfloat16 with round-to-nearest-even.  The GEMM-optimisation
 * article at www.lqnn.cn (news/123226), section 2.2, defines the format (8
 * exponent and 7 fraction bits, FP32's range) and the bf16 x bf16 product
 * accumulated in FP32.  Arguments, layout, ownership, degenerate sizes and
 * errors exactly as gemm_nt_f16.
 */
int gemm_nt_bf16(const void *A, const void *B, void *D,
                 int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * The fp16 product with an fp16 running sum instead of fp32 (the f16
 * accumulator of page "如何用 Croqtile 一步步优化矩阵乘法内核", sections
 * "内核 0：朴素版" and "内核 2：Hopper TMA + WGMMA", which notes that it takes
 * fewer registers):
 *
 *     s = +0;  for each chunk c of 64 consecutive k (the chunks aligned to
 *     K's end, so the first holds the K mod 64 leading terms when K is not a
 *     multiple of 64):  s = fp16(s + fp16(sum_{k in c} A[m,k] * B[n,k]));
 *     D[m,n] = s
 *
 * Each chunk's products are summed in fp32 by the matrix unit, the sum is
 * rounded to fp16 and added to s with an fp16 addition (both roundings to
 * nearest even), so partial sums above 2048 lose integer precision and
 * errors grow with the number of chunks.  D is never -0.
 * Arguments, layout, ownership, degenerate sizes and errors exactly as
 * gemm_nt_f16.
 */
int gemm_nt_f16_acc16(const void *A, const void *B, void *D,
                      int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * Host-only introspection of gemm_nt_f16_acc16: the output tile (*bm x *bn)
 * and load mode (*lbytes: 16 = 16-byte direct-to-LDS loads, 1 =
 * register-staged chunks) a call with these pointers and sizes runs.
 * A and B are only inspected for alignment, never dereferenced.  Returns
 * GEMM_OK, or GEMM_EINVAL for a size out of the entry points' range or a
 * NULL output pointer.
 */
int gemm_nt_f16_acc16_kernel(const void *A, const void *B, int64_t M, int64_t N, int64_t K,
                             int *bm, int *bn, int *lbytes);

/* FP8 operand formats (OCP 8-bit floating point). */
#define GEMM_FP8_E4M3 0  /* 1 sign, 4 exponent (bias 7), 3 fraction bits; S.1111.111
                            is NaN; no infinities; largest finite 448            */
#define GEMM_FP8_E5M2 1  /* 1 sign, 5 exponent (bias 15), 2 fraction bits; IEEE-style
                            infinities and NaNs; largest finite 57344             */

/*
 * FP8 product with a per-tensor scale (the GEMM-optimisation article at
 * www.lqnn.cn, news/123226: section 2.2 names the E4M3 and E5M2 formats,
 * sections 4.2-4.3 quantise each operand with a scale kept in fp32 and undo
 * it after an fp32-accumulated product):
 *
 *     D[m,n] = scale * sum_{k<K} A[m,k] * B[n,k]
 *
 * A: M x K bytes in a_format, B: N x K bytes in b_format (GEMM_FP8_E4M3 or
 *   GEMM_FP8_E5M2, chosen per operand), both row-major with no padding,
 *   any alignment.  D: M x N fp16, 2-byte aligned.
 * scale: fp32, normally the product of A's and B's dequantisation scales.
 *   Products are exact and summed in fp32; the sum is multiplied by scale in
 *   fp32 and rounded once to fp16 (round to nearest even).  K == 0 gives
 *   scale * (+0).
 * Load paths: 16-byte loads straight into LDS when K % 16 == 0 with A and
 *   B 16-byte aligned, and when K is even (K >= 16) with A and B 2-byte
 *   aligned and M, N > 64; then 4 bytes per lane when K % 4 == 0 with
 *   4-byte alignment; anything else loads 16-byte chunks into registers at
 *   any alignment and writes them to LDS (128 x 128 or 64 x 64 tiles), all
 *   on the FP8 MFMA.
 *
 * Returns as gemm_nt_f16 (sizes M, N, K in [0, 2^31 - 1], K <= GEMM_MAX_K),
 * and GEMM_EINVAL also for an unknown format or D overlapping A or B.
 */
int gemm_nt_fp8(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                float scale, int a_format, int b_format, hipStream_t stream);

/*
 * FP8 product with per-channel weight scales (the same article, section 4.2:
 * weights are quantised with one scale per output channel, the largest
 * magnitude of each weight row over 448, activations with one scale per
 * tensor).  B holds the weights, so row n of B is output channel n:
 *
 *     D[m,n] = (a_scale * b_scale[n]) * sum_{k<K} A[m,k] * B[n,k]
 *
 * A, B, D, formats and the fast path as gemm_nt_fp8.
 * a_scale: fp32, A's dequantisation scale.  b_scale: device pointer to N
 *   fp32 values (B's per-row dequantisation scales), 4-byte aligned, read
 *   only, owned by the caller; it may be NULL only when M or N is 0.  The
 *   factor a_scale * b_scale[n] is formed in fp32 (round to nearest even),
 *   then multiplies the fp32 sum, and the result is rounded once to fp16.
 *   K == 0 gives (a_scale * b_scale[n]) * (+0).
 *
 * Returns as gemm_nt_fp8, and GEMM_EINVAL also for a NULL or misaligned
 * b_scale, or D overlapping b_scale.
 */
int gemm_nt_fp8_cs(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                   float a_scale, const float *b_scale, int a_format, int b_format,
                   hipStream_t stream);

/*
 * Host-only: the output tile gemm_nt_fp8 uses for these sizes (aligned16:
 * whether A and B are 16-byte aligned; 4-byte alignment is assumed
 * otherwise), following the load paths above.
 * GEMM_EINVAL for sizes out of the entry points' range or NULL outputs.
 */
int gemm_nt_fp8_tile(int64_t M, int64_t N, int64_t K, int aligned16, int *bm, int *bn);

/*
 * Fused epilogue, the standard GEMM form (the GEMM-optimisation article at
 * www.lqnn.cn, news/123226, section 2.1, writes GEMM as C = alpha*A*B +
 * beta*C; its section 3.4 builds the same alpha/beta combination into the
 * kernel's epilogue; the per-column bias is a linear layer's):
 *
 *     D[m,n] = alpha * sum_{k<K} A[m,k] * B[n,k] + beta * C[m,n] + bias[n]
 *
 * The product is the one gemm_nt_f16 computes (fp32 accumulation); the
 * epilogue is formed in fp32 in the order written and rounded once to fp16
 * (round to nearest even).  bias holds one value per output column, as a
 * linear layer's bias does.
 *
 * C: M x N fp16, row-major, read only when beta != 0 (it may then be NULL
 *   otherwise); it may be D itself (in place) but must not otherwise overlap
 *   D.  bias: N fp16 values or NULL (no bias); must not overlap D.
 * alpha, beta: fp32 scalars.  alpha == 1, beta == 0 and no bias is exactly
 *   gemm_nt_f16.  K == 0 gives alpha * (+0) + beta * C + bias.
 *
 * Returns as gemm_nt_f16, and GEMM_EINVAL also for beta != 0 with a NULL C,
 * C or bias not 2-byte aligned, C overlapping D without being D, or bias
 * overlapping D.
 */
int gemm_nt_f16_ex(const void *A, const void *B, const void *C, const void *bias, void *D,
                   int64_t M, int64_t N, int64_t K, float alpha, float beta,
                   hipStream_t stream);

/*
 * Stream-K form of gemm_nt_f16 for shapes whose tiles do not fill whole
 * waves of the GPU's CUs (page 2, "构建 Tiled GEMM", names persistent kernels
 * with a software pipeline as the next step after its tiled kernel; page 1
 * notes that persistent kernels amortise launch costs at large sizes).  The
 * result is D = A * B^T exactly as gemm_nt_f16 defines it; only the order of
 * the fp32 additions differs, and it is fixed for a given shape, so repeated
 * calls are bitwise identical.
 *
 * A persistent grid of one workgroup per CU (at most 256) splits the
 * K-steps of the tiles evenly over all workgroups; a tile split over several
 * workgroups is summed in fp32 through `workspace` and rounded to fp16 once.
 * It is used (P = the GPU's CUs, K-steps of 64):
 *   - M and N > 64: on 128 x 128 tiles when those fill at most P/4 and K
 *     spans at least 192 steps (K > 12224);
 *   - M or N <= 64 with K % 8 == 0 (16-byte aligned rows): on 64 x 64 tiles
 *     when there are P/4 to P/2 of them and either the plain grid's 64 x 32
 *     (or 32 x 64) tiles number fewer than P or K spans at least 128 steps;
 *     else on the plain grid's tile when those fill at most P/2 and the
 *     workgroups get at least 8 steps each; in both cases K spans at least
 *     64 steps (K > 4032).
 * Other shapes run exactly as gemm_nt_f16.
 *
 * workspace: device memory of at least gemm_nt_f16_ws_size(M, N, K) bytes,
 *   256-byte aligned, not overlapping A, B or D, owned by the caller.  It
 *   must be zero-filled before its first use; every call leaves it ready for
 *   the next one, so it is reused without clearing, for any shape.  Its first
 *   256 bytes are a header: the 32-bit word at byte offset 0 counts calls
 *   (each call's flags carry that call's number, so a flag left by an earlier
 *   call never counts as raised), the word at offset 4 is zero between
 *   calls, and the word at offset 8 becomes nonzero when a wait timed out
 *   (below); it stays set until the caller zeroes it.  Calls that share a
 *   workspace must not run concurrently (order them on one stream).
 * ws_bytes: its size in bytes.  When the shape does not benefit from
 *   stream-K, or ws_bytes is too small for the plan, the call runs exactly
 *   as gemm_nt_f16 (workspace unused; it may then be NULL with ws_bytes 0).
 *
 * All workgroups of the grid must be resident at once: the call expects the
 * GPU's CUs not to be held by other long-running work, which includes
 * another stream-K call (of this entry point or gemm_nt_f16_ws_noalloc),
 * even with its own workspace: order stream-K calls on one stream.  A workgroup that
 * waits more than ~5 s for another writes its tile as NaN (0x7E00), sets the
 * header's error word and ends, so the kernel always terminates; the
 * workspace stays valid for later calls.
 *
 * Returns GEMM_OK, GEMM_EINVAL (as gemm_nt_f16, or ws_bytes < 0, a NULL or
 * misaligned workspace with ws_bytes > 0, or a workspace overlapping A, B or
 * D) or GEMM_ELAUNCH.
 */
int gemm_nt_f16_ws(const void *A, const void *B, void *D,
                   int64_t M, int64_t N, int64_t K,
                   void *workspace, int64_t ws_bytes, hipStream_t stream);

/*
 * gemm_nt_f16_ws without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It computes exactly what gemm_nt_f16_ws
 * computes, with the same plan, kernels and results, and calls no allocating
 * routine: the workspace is a static device array of the library (16 MiB +
 * 1.25 KiB per GPU, loaded with the library's code and held until the
 * process ends), looked up once per device on the first call, which also
 * enqueues a small kernel that zeroes its header and flags.
 *
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or different threads, without ordering) race and give
 * wrong results; order them on one stream.  A wait that times out behaves as
 * in gemm_nt_f16_ws (NaN tile; the error word is in the static array, not
 * readable by the caller).
 *
 * Arguments as gemm_nt_f16.  Returns GEMM_OK, GEMM_EINVAL (as gemm_nt_f16),
 * GEMM_ESCRATCH (the plan needs more workspace than the static array holds;
 * not reached on GPUs of up to 256 CUs) or GEMM_ELAUNCH (also when the
 * array's device address cannot be obtained).
 */
int gemm_nt_f16_ws_noalloc(const void *A, const void *B, void *D,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * Host-only (no HIP call): bytes of workspace gemm_nt_f16_ws needs for this
 * shape with operands aligned to 16 bytes (0: it would not use stream-K).
 * Sizes out of range give 0.
 */
int64_t gemm_nt_f16_ws_size(int64_t M, int64_t N, int64_t K);

/*
 * Host-only introspection (no HIP call) of gemm_nt_f16_ws's plan for 16-byte
 * aligned operands on 256 CUs: the tile, the workgroups launched and how
 * many tiles are split by K-steps (0: the plain one-workgroup-per-tile
 * launch).  Returns GEMM_OK or GEMM_EINVAL (a size out of the entry
 * points' range, or a NULL output).
 */
int gemm_nt_f16_ws_tile(int64_t M, int64_t N, int64_t K, int *bm, int *bn,
                        int64_t *workgroups, int64_t *sk_tiles);

/*
 * Host-only (no HIP call): the work items workgroup `wg` runs under that
 * plan, in order, 5 values each: tile, first K-step, end K-step (K-steps
 * of 64), and the first and last workgroup whose partial sums it adds (none
 * when first > last).  A first K-step > 0 means the workgroup only
 * contributes a partial sum to that tile.  Writes at most max_items items
 * to `items` and the full count to *count (0 when the plan is not
 * stream-K).  Tiles are numbered as gemm_nt_f16_tile_coord maps them.
 * Returns GEMM_OK or GEMM_EINVAL (sizes out of range, wg outside the grid,
 * NULL outputs).
 */
int gemm_nt_f16_ws_items(int64_t M, int64_t N, int64_t K, int64_t wg,
                         int64_t *items, int64_t max_items, int64_t *count);

/* Static text for a return code; never NULL. */
const char *gemm_nt_f16_strerror(int code);

/*
 * Host-only introspection (no HIP call): the output tile BM x BN and the K
 * step BK that gemm_nt_f16 uses for an M x N x K problem with operands
 * aligned to 16 bytes, and the number of workgroups it launches.  Tests use
 * it to pick rows and columns at tile edges.  Returns GEMM_OK or GEMM_EINVAL
 * (a size out of the entry points' range, or a NULL output).
 */
int gemm_nt_f16_tile(int64_t M, int64_t N, int64_t K,
                     int *bm, int *bn, int *bk, int64_t *workgroups);

/*
 * Host-only introspection (no HIP call) of the kernel a gemm_nt_f16 call
 * with these pointers and sizes takes (gemm_nt_bf16 and gemm_nt_f16_ex take
 * the same one): the output tile *bm x *bn; *load_bytes, how operand chunks
 * reach LDS (16: 16-byte loads straight into LDS, at any 2-byte alignment,
 * when K % 8 == 0 with A and B 16-byte aligned, and otherwise when K >= 8
 * and M, N > 64; 1: 16-byte loads into registers, then LDS writes, for
 * K < 8 and for M or N <= 64 with rows not 16-byte aligned); *store, the
 * epilogue's store form (0: element
 * stores; 1: 8-byte stores, D 8-byte aligned and N % 4 == 0; 2: whole tiles
 * staged through LDS and written with 16-byte stores, D 16-byte aligned and
 * N % 8 == 0).  (The 256 x 256 tile with 16-byte loads keeps A in two LDS
 * stages and B in three when K % 512 != 0, in two otherwise.)  The pointers
 * are only inspected, never dereferenced.
 * Returns GEMM_OK or GEMM_EINVAL (a size out of the entry points' range, or
 * a NULL output).
 */
int gemm_nt_f16_kernel(const void *A, const void *B, const void *D,
                       int64_t M, int64_t N, int64_t K,
                       int *bm, int *bn, int *load_bytes, int *store);

/*
 * Host-only introspection (no HIP call): the output tile (tile_m, tile_n)
 * that workgroup `wg` computes when the output is split into tiles_m x
 * tiles_n tiles (each count in [1, 2^31 - 1]).  The map is a bijection of
 * [0, tiles_m*tiles_n) onto the tiles; it keeps tiles that share A or B rows
 * on the same L2 slice.  Returns GEMM_OK or GEMM_EINVAL (wg or a count out
 * of range, NULL output).
 */
int gemm_nt_f16_tile_coord(int64_t wg, int64_t tiles_m, int64_t tiles_n,
                           int64_t *tile_m, int64_t *tile_n);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_NT_F16_H */
