/*
 * sgemm_mi355 -- single-precision matrix multiply for AMD Instinct MI355X
 * (gfx950, CDNA4), C = A.B on row-major FP32 matrices with FP32 accumulation.
 *
 * The operation. Element (i, j) of C is the dot product of row i of A and
 * column j of B: C[i][j] = sum_{k<K} A[i][k] * B[k][j], one multiply and one
 * add per term, 2*M*N*K floating-point operations per call (ratcatcher.ru
 * "Matrix multiplication: naive and tiled", section 1; GPU Parallel Book
 * ch. 9 "Optimised Matrix Multiplication", section 9.1). Matrices are stored
 * row by row, element (row, col) at offset row*ld + col (ratcatcher page,
 * section 1); general M, N, K follow the CUDA Handbook, ch. 17, section 17.3.
 * The scale factors are fixed: alpha = 1, beta = 0, so C is written, never
 * read.
 *
 * Layout of every call:
 *   A: M x K, element (i, k) at A[(size_t)i*lda + k], lda >= max(1, K)
 *   B: K x N, element (k, j) at B[(size_t)k*ldb + j], ldb >= max(1, N)
 *   C: M x N, element (i, j) at C[(size_t)i*ldc + j], ldc >= max(1, N)
 *   Columns j in [N, ldc) of C (row padding) are never written; padding of A
 *   and B is never used in a result.
 *
 * Ownership and execution. A, B and C are device pointers owned by the
 * caller; `stream` is the caller's HIP stream (0 = the default stream). A
 * call validates its arguments on the host, enqueues one kernel on `stream`
 * and returns without synchronising; results are visible to work ordered
 * after it on that stream. The library allocates no memory and never
 * synchronises the device; its only mutable global state is the per-device
 * address of the static scratch of sgemm_mi355_splitk_noalloc, looked up
 * once under a lock (calls are thread-safe).
 * A kernel fault surfaces at the caller's next synchronisation.
 *
 * Precision. Products and sums are FP32 (CDNA4 FP32 matrix instructions in
 * the main path, FP32 fused multiply-add in the vector path); nothing is
 * converted to a narrower type. The summation order differs from a plain
 * k-ascending loop, so results agree with one to within
 * |C - C_exact| <= 4*K*2^-23*sum_k |A[i][k]*B[k][j]| per element; inputs whose
 * partial sums are integers below 2^24 give exact results.
 *
 * Errors. Every entry point returns SGEMM_MI355_OK (0) or a negative code.
 * Argument errors are detected on the host before any HIP call; nothing is
 * enqueued then. No entry point aborts or throws.
 */
#ifndef SGEMM_MI355_H
#define SGEMM_MI355_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_MI355_OK 0
#define SGEMM_MI355_ERR_DIM (-1)      /* M, N or K is negative */
#define SGEMM_MI355_ERR_LD (-2)       /* lda < max(1,K), ldb < max(1,N) or ldc < max(1,N) */
#define SGEMM_MI355_ERR_NULL (-3)     /* a null pointer for a matrix with elements */
#define SGEMM_MI355_ERR_ALIAS (-4)    /* C's extent overlaps A's or B's */
#define SGEMM_MI355_ERR_EXTENT (-5)   /* the tile grid exceeds one launch's limits */
#define SGEMM_MI355_ERR_LAUNCH (-6)   /* the HIP runtime rejected the launch */
#define SGEMM_MI355_ERR_CONFIG (-7)   /* unknown kernel configuration id */
#define SGEMM_MI355_ERR_ALIGN (-8)    /* a pointer is not 4-byte aligned */
#define SGEMM_MI355_ERR_STRIDE (-9)   /* a batch stride is negative, or batch entries of C overlap */
#define SGEMM_MI355_ERR_OP (-10)      /* an op argument is neither OP_N nor OP_T */
#define SGEMM_MI355_ERR_WORKSPACE (-11) /* split-K or stream-K workspace smaller than required */
#define SGEMM_MI355_ERR_SCRATCH (-12) /* split-K partial sums larger than SGEMM_MI355_SCRATCH_BYTES */

/* Size of the library's static device scratch (per device), used only by
 * sgemm_mi355_splitk_noalloc. */
#define SGEMM_MI355_SCRATCH_BYTES (32u << 20)

/* Operand ops for the general entry points (row-major storage throughout). */
#define SGEMM_MI355_OP_N 0 /* op(X) = X */
#define SGEMM_MI355_OP_T 1 /* op(X) = X^T */

/*
 * Main entry point: C = A.B with the kernel configuration the built-in
 * selection picks for (M, N, K): measured run times of the configurations on
 * a grid of shapes, carried to other shapes by a model of how their
 * workgroups fill the compute units (tile sizes chosen by measurement, as the
 * CUDA Handbook section 17.3 and GPU Parallel Book section 9.6 prescribe).
 * Quick returns: M == 0 or N == 0 does nothing and returns 0; K == 0 sets the
 * M x N block of C to +0 (the empty sum). Any 4-byte-aligned pointers and any
 * leading dimensions allowed above are accepted.
 */
int sgemm_mi355(int M, int N, int K,
                const float *A, int lda,
                const float *B, int ldb,
                float *C, int ldc,
                hipStream_t stream);

/*
 * Same contract as sgemm_mi355, computed by the vector-FMA comparison kernel
 * (LDS-tiled register microtile, in the spirit of the register-tiled kernel of
 * GPU Parallel Book section 9.5 and the 8x8 microtile of the CUDA Handbook
 * section 17.3) instead of the matrix-core path.
 */
int sgemm_mi355_valu(int M, int N, int K,
                     const float *A, int lda,
                     const float *B, int ldb,
                     float *C, int ldc,
                     hipStream_t stream);

/*
 * Same contract, with the kernel configuration forced to `config`
 * (0 <= config < sgemm_mi355_num_configs()); returns SGEMM_MI355_ERR_CONFIG
 * for an unknown id. Used to measure every configuration (tile tuning) and to
 * test each one, not only those the table picks.
 */
int sgemm_mi355_with_config(int M, int N, int K,
                            const float *A, int lda,
                            const float *B, int ldb,
                            float *C, int ldc,
                            hipStream_t stream, int config);

/*
 * General product, the BLAS form of the same operation:
 *   C = alpha * op(A) . op(B) + beta * C,
 * op(A) M x K and op(B) K x N, all matrices row-major:
 *   opA = OP_N: A is M x K, element (i, k) at A[i*lda + k], lda >= max(1, K);
 *   opA = OP_T: A is K x M, op(A)(i, k) = A[k*lda + i],     lda >= max(1, M);
 *   opB = OP_N: B is K x N, element (k, j) at B[k*ldb + j], ldb >= max(1, N);
 *   opB = OP_T: B is N x K, op(B)(k, j) = B[j*ldb + k],     ldb >= max(1, K).
 * The product is the dot-product definition of the pages (see above); the
 * scale factors extend it the way the BLAS interface does. When beta == 0, C
 * is not read (NaN in C does not propagate). When alpha == 0 or K == 0, A and
 * B are not read and C = beta * C. The product is rounded to FP32, scaled by
 * alpha, and then beta * C is added with one fused multiply-add.
 * Errors as above, plus SGEMM_MI355_ERR_OP for an op other than OP_N/OP_T.
 */
int sgemm_mi355_ex(int opA, int opB, int M, int N, int K, float alpha,
                   const float *A, int lda, const float *B, int ldb,
                   float beta, float *C, int ldc, hipStream_t stream);

/*
 * Strided batch of independent general products in one launch:
 *   C_b = alpha * op(A_b) . op(B_b) + beta * C_b,  b = 0 .. batch-1,
 * with A_b = A + b*strideA, B_b = B + b*strideB, C_b = C + b*strideC
 * (strides in elements). strideA or strideB may be 0 (one operand shared by
 * every product); strides are never negative, and when batch > 1 strideC
 * must keep the C_b apart (strideC >= (M-1)*ldc + N), else
 * SGEMM_MI355_ERR_STRIDE. batch == 0 does nothing; a negative batch is
 * SGEMM_MI355_ERR_DIM. C may not overlap any A_b or B_b. The batch is a second
 * grid dimension, so many small products fill the chip together.
 */
int sgemm_mi355_strided_batched(int opA, int opB, int M, int N, int K, float alpha,
                                const float *A, int lda, long long strideA,
                                const float *B, int ldb, long long strideB,
                                float beta, float *C, int ldc, long long strideC,
                                int batch, hipStream_t stream);

/*
 * sgemm_mi355_strided_batched with the kernel configuration forced to
 * `config`, which must have been built for this (opA, opB) pair
 * (sgemm_mi355_config_ops), else SGEMM_MI355_ERR_CONFIG. For tuning and
 * tests.
 */
int sgemm_mi355_strided_batched_with_config(int opA, int opB, int M, int N, int K, float alpha,
                                            const float *A, int lda, long long strideA,
                                            const float *B, int ldb, long long strideB,
                                            float beta, float *C, int ldc, long long strideC,
                                            int batch, hipStream_t stream, int config);

/*
 * Split-K form of sgemm_mi355_ex for problems whose M x N grid of block tiles
 * is too small to fill the chip: K is cut into up to `splits` chunks (each a
 * multiple of 32 values of k, the last one taking the rest; fewer chunks when
 * K is small). Chunk s writes op(A)[:, chunk s] . op(B)[chunk s, :] into a
 * dense M x N FP32 partial (row stride N) in `workspace`; a second kernel then
 * sets C = alpha * (sum of the partials, added in ascending chunk order) +
 * beta * C. The fixed order makes the result independent of timing (repeated
 * calls give identical bits); it rounds differently from the unsplit product
 * but stays within the same error bound, and integer-valued products are
 * exact. `workspace` is device memory owned by the caller, at least
 * sgemm_mi355_splitk_workspace_size(M, N, K, splits) bytes, 4-byte aligned,
 * not overlapping A, B or C; it is not needed (may be NULL) when that size is
 * 0. Both kernels are enqueued on `stream`; the workspace may be reused once
 * work ordered after them on that stream starts. 1 <= splits <= 256, else
 * SGEMM_MI355_ERR_DIM; a short workspace gives SGEMM_MI355_ERR_WORKSPACE.
 */
int sgemm_mi355_splitk(int opA, int opB, int M, int N, int K, float alpha,
                       const float *A, int lda, const float *B, int ldb,
                       float beta, float *C, int ldc, int splits,
                       float *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sgemm_mi355_splitk for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that forbid allocation, harnesses
 * that forbid hipMalloc): the same computation, the same split plan and the
 * same kernels, so the same bits, but the partial sums go to a static device
 * array of SGEMM_MI355_SCRATCH_BYTES that the library holds on every device
 * it runs on until the process ends, instead of a caller workspace. The call
 * allocates nothing (no hipMalloc, no allocating library routine); its first
 * call on a device looks the array's device address up once. Every call on
 * one device shares that device's array: calls whose work overlaps on one
 * device (different streams, or threads racing on one stream's enqueue order)
 * race on it and must be ordered by the caller; calls ordered on one stream
 * are safe. Nothing in the array needs clearing: every partial sum is
 * written before it is read. Errors as sgemm_mi355_splitk, plus
 * SGEMM_MI355_ERR_SCRATCH when 4 * chunks * M * N bytes of partial sums
 * (sgemm_mi355_splitk_workspace_size) exceed SGEMM_MI355_SCRATCH_BYTES;
 * nothing is enqueued then.
 */
int sgemm_mi355_splitk_noalloc(int opA, int opB, int M, int N, int K, float alpha,
                               const float *A, int lda, const float *B, int ldb,
                               float beta, float *C, int ldc, int splits, hipStream_t stream);

/* Workspace bytes sgemm_mi355_splitk needs (0: no split, none needed). */
size_t sgemm_mi355_splitk_workspace_size(int M, int N, int K, int splits);

/*
 * sgemm_mi355_splitk with the tile configuration of the chunk products
 * forced to `config` (built for this opA/opB pair). For tuning and tests.
 */
int sgemm_mi355_splitk_with_config(int opA, int opB, int M, int N, int K, float alpha,
                                   const float *A, int lda, const float *B, int ldb,
                                   float beta, float *C, int ldc, int splits,
                                   float *workspace, size_t workspace_bytes,
                                   hipStream_t stream, int config);

/*
 * Split count and tile configuration the library suggests for a problem
 * (host only). Within a factor of two (in each of M, N, K) of the measured
 * split-K grid (M, N from 64 to 2048, K from 1024 to 65536, powers of two),
 * the fastest split count measured at the nearest grid shape. Elsewhere: no
 * split while the unsplit tile grid gives at least two workgroups per compute
 * unit, otherwise the largest power of two that keeps chunks of at least 1024
 * values of k. The count is then cut into chunks as sgemm_mi355_splitk does
 * (multiples of 32 values of k). Writes *splits and *config (the
 * configuration of the chunk products, or of the whole product when *splits
 * is 1). Returns 0, or SGEMM_MI355_ERR_OP / SGEMM_MI355_ERR_DIM / _NULL for
 * bad arguments.
 */
int sgemm_mi355_select_splitk(int opA, int opB, int M, int N, int K, int *splits, int *config);

/*
 * Stream-K form of sgemm_mi355_ex (single products), for large problems whose
 * tile count leaves the last round of workgroups thin (the work-centric
 * decomposition of Osama et al., PPoPP 2023). A persistent grid of
 * (compute units x occupancy) workgroups runs the whole rounds of block tiles
 * as sgemm_mi355_ex does, and deals the BK-deep slabs of the remaining tiles
 * out evenly, in contiguous ranges that cross tile boundaries. A tile split
 * between workgroups leaves dense BM x BN blocks of partial sums in
 * `workspace`; a second kernel adds them in ascending k order and sets
 * C = alpha * sum + beta * C. The order is fixed, so repeated calls on one
 * device give identical bits; the result rounds differently from the unsplit
 * product but stays within the same error bound, and integer-valued products
 * are exact.
 *
 * The library picks the configuration with a model of the measured table
 * (sgemm_mi355_select_streamk) and runs the plain sgemm_mi355_ex path where
 * stream-K is not predicted to pay. `workspace` is device memory owned by the
 * caller, at least sgemm_mi355_streamk_workspace_size(opA, opB, M, N, K, -1)
 * bytes (it depends on the current device's compute units), 16-byte aligned,
 * not overlapping A, B or C; it may be NULL when that size is 0. Both kernels
 * are enqueued on `stream`; the workspace may be reused once work ordered
 * after them on that stream starts. A short workspace gives
 * SGEMM_MI355_ERR_WORKSPACE, a misaligned one SGEMM_MI355_ERR_ALIGN; the
 * other errors are those of sgemm_mi355_ex.
 */
int sgemm_mi355_streamk(int opA, int opB, int M, int N, int K, float alpha,
                        const float *A, int lda, const float *B, int ldb,
                        float beta, float *C, int ldc,
                        float *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sgemm_mi355_streamk with configuration `config`, which must have a
 * stream-K form (sgemm_mi355_config_streamk) built for this opA/opB pair,
 * else SGEMM_MI355_ERR_CONFIG. When the tiles fill whole rounds of the grid,
 * nothing is split: it runs the plain launch of `config` and needs no
 * workspace. For tuning and tests.
 */
int sgemm_mi355_streamk_with_config(int opA, int opB, int M, int N, int K, float alpha,
                                    const float *A, int lda, const float *B, int ldb,
                                    float beta, float *C, int ldc,
                                    float *workspace, size_t workspace_bytes,
                                    hipStream_t stream, int config);

/*
 * Workspace bytes the stream-K call needs on the current device: for
 * configuration `config`, or with config = -1 for the library's own choice
 * (either operand alignment). Two BM x BN FP32 blocks per workgroup of the
 * grid (128 MiB for 256 x 256 tiles on 256 compute units); 0 when no tile
 * is split, or for invalid arguments.
 */
size_t sgemm_mi355_streamk_workspace_size(int opA, int opB, int M, int N, int K, int config);

/*
 * The configuration sgemm_mi355_streamk would run in stream-K form for
 * 16-byte aligned operands, or -1 when it would take the plain path (host
 * only). Returns 0, or SGEMM_MI355_ERR_OP / _DIM / _NULL.
 */
int sgemm_mi355_select_streamk(int opA, int opB, int M, int N, int K, int *config);

/* 1 if configuration `config` has a stream-K form, 0 if not, or SGEMM_MI355_ERR_CONFIG. */
int sgemm_mi355_config_streamk(int config);

/*
 * Argument validation alone: returns the code the entry points above would
 * return for these arguments before touching the GPU (0 if they would run).
 * Pure host code; makes no HIP call.
 */
int sgemm_mi355_validate(int M, int N, int K,
                         const float *A, int lda,
                         const float *B, int ldb,
                         const float *C, int ldc);

/*
 * Validation of the general/batched arguments alone (pure host code, no HIP
 * call): the code sgemm_mi355_strided_batched would return before launching.
 */
int sgemm_mi355_validate_ex(int opA, int opB, int M, int N, int K, float alpha,
                            const float *A, int lda, long long strideA,
                            const float *B, int ldb, long long strideB,
                            float beta, const float *C, int ldc, long long strideC, int batch);

/*
 * Configuration id the selection picks for a plain single product of this
 * shape (host only), assuming 16-byte aligned operands with leading
 * dimensions that are multiples of 4; sgemm_mi355 itself checks the actual
 * pointers and may pick a register-staged configuration for others.
 */
int sgemm_mi355_select_config(int M, int N, int K);

/*
 * Configuration id sgemm_mi355 runs for exactly these arguments (host only):
 * the selection above with the alignment of the actual pointers and leading
 * dimensions taken into account (16-byte aligned A and B with lda and ldb
 * multiples of 4 may take a direct-to-LDS configuration, others take a
 * register-staged one). The pointers are only inspected, never read.
 * Returns SGEMM_MI355_ERR_DIM for a negative dimension.
 */
int sgemm_mi355_selected_config(int M, int N, int K, const float *A, int lda, const float *B, int ldb);

/*
 * How configuration `config` stages the slabs of a single product with these
 * arguments (host only; the pointers are only inspected): 0 through
 * registers, 1 by direct global-to-LDS loads, 2 by direct loads for the
 * whole slabs and through registers for a partial last slab (K not a multiple
 * of the slab depth). Direct loads need 16-byte aligned A and B, leading
 * dimensions that are multiples of 4, K of at least one slab and, for an
 * operand whose rows run along M or N (B, or A transposed), that extent a
 * multiple of 4. A and B are in the layouts the configuration reads
 * (sgemm_mi355_config_ops). Returns SGEMM_MI355_ERR_CONFIG for an unknown id,
 * SGEMM_MI355_ERR_DIM for a negative dimension.
 */
int sgemm_mi355_config_staging(int config, int M, int N, int K, const float *A, int lda, const float *B, int ldb);

/* Configuration id sgemm_mi355_valu uses for a problem shape (host only). */
int sgemm_mi355_select_config_valu(int M, int N, int K);

/*
 * Configuration id chosen for a general or batched problem (host only), with
 * the same alignment assumption as sgemm_mi355_select_config.
 */
int sgemm_mi355_select_config_ex(int opA, int opB, int M, int N, int K, int batch);

/*
 * Operand ops a configuration was built for: writes OP_N/OP_T through the
 * non-null pointers; returns 0 or SGEMM_MI355_ERR_CONFIG.
 */
int sgemm_mi355_config_ops(int config, int *opA, int *opB);

/* Number of kernel configurations compiled into the library. */
int sgemm_mi355_num_configs(void);

/*
 * Static description of configuration `config`: a NUL-terminated string such
 * as "mfma32_256x256x16_w2x2" (kernel kind, block tile BMxBNxBK, waves), or
 * NULL for an unknown id. The string is owned by the library.
 */
const char *sgemm_mi355_config_name(int config);

/*
 * Tile geometry of configuration `config`: writes the block tile rows (bm),
 * columns (bn), K-slab depth (bk) and threads per workgroup (threads) through
 * the non-null pointers; returns 0 or SGEMM_MI355_ERR_CONFIG.
 */
int sgemm_mi355_config_info(int config, int *bm, int *bn, int *bk, int *threads);

/*
 * Workgroups of configuration `config` that one compute unit of the current
 * device holds at once (hipOccupancyMaxActiveBlocksPerMultiprocessor for the
 * kernel the configuration runs on 16-byte aligned operands, at its
 * workgroup size): writes it through `workgroups_per_cu`. Returns 0,
 * SGEMM_MI355_ERR_CONFIG for an unknown id, SGEMM_MI355_ERR_NULL for a null
 * pointer, or SGEMM_MI355_ERR_LAUNCH when the HIP runtime cannot answer (no
 * device). Needs a GPU; enqueues nothing. The tuner records it next to its
 * timings for the selection's model of partly filled waves.
 */
int sgemm_mi355_config_occupancy(int config, int *workgroups_per_cu);

/*
 * Diagnostic: the workgroup -> C-tile map every kernel uses. For workgroup
 * `bid` of a tiles_m x tiles_n grid of block tiles walked in bands of
 * `group_m` tile rows, writes the tile row (*tm) and column (*tn). Workgroups
 * are renumbered so consecutive logical ids share one of the 8 XCDs (and its
 * L2). The map is a bijection on [0, tiles_m*tiles_n). Returns 0, or
 * SGEMM_MI355_ERR_DIM for out-of-range arguments. Pure host code.
 */
int sgemm_mi355_tile_map(int bid, int tiles_m, int tiles_n, int group_m, int *tm, int *tn);

/* Static message for an error code (never NULL). */
const char *sgemm_mi355_strerror(int code);

/* Library version string, e.g. "0.6.1". */
const char *sgemm_mi355_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_MI355_H */
