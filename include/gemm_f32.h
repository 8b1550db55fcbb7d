/*
 * gemm_f32.h -- C ABI of the MI355X (gfx950) fp32 matrix-multiply library.
 *
 * The operation is the dense product C = A x B in fp32 that the pages build
 * their kernels for: each output element is the dot product of a row of A
 * with a column of B along the shared K dimension (ijyty.com tiled-matmul
 * article, naive-review paragraph; mayulu.co "CUDA 编程系列之三", section 6).
 * The pages show only kernels over square N x N row-major matrices with
 * leading dimension N (geek-doc.cn "矩阵乘法 tiling", sections 一 and 四); this
 * interface generalises that to M x K times K x N with explicit leading
 * dimensions and keeps the pages' "C is assigned, never accumulated into".
 *
 * Layout (all matrices row-major, element type float, 4-byte aligned):
 *   A[i][k] = A[i*lda + k]  for 0 <= i < M, 0 <= k < K
 *   B[k][j] = B[k*ldb + j]  for 0 <= k < K, 0 <= j < N
 *   C[i][j] = C[i*ldc + j]  for 0 <= i < M, 0 <= j < N
 * Result: C[i][j] = sum_{k<K} A[i][k] * B[k][j], accumulated in fp32 in an
 * order that depends on the variant (several fp32 results are correct for
 * non-integer inputs; integer-valued inputs whose partial sums stay below
 * 2^24 give the exact result on every variant).  Elements of C outside the
 * M x N window (the ldc padding) are never written.
 *
 * Memory and ownership: A, B and C are device pointers owned by the caller
 * (for example the storage of torch tensors).  The library allocates no
 * device memory, keeps no per-call state, and is re-entrant, with one
 * exception: gemm_f32_splitk_noalloc keeps its split-K slabs in a fixed
 * device array of the library (see there).  C must not overlap A or B.
 *
 * Streams: `stream` is a hipStream_t passed as void*; NULL means the null
 * stream.  Calls are asynchronous: they return once the kernel is enqueued.
 * Argument errors are returned synchronously before anything is enqueued;
 * launch errors are the launch call's own status (see gemm_f32_last_error); faults
 * during execution surface at the caller's next synchronisation.
 */
#ifndef GEMM_F32_H
#define GEMM_F32_H

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes --------------------------------------------------- */
#define GEMM_F32_OK 0
#define GEMM_F32_INVALID_DIM 1   /* M, N or K negative                      */
#define GEMM_F32_INVALID_LD 2    /* lda < max(1,K), ldb or ldc < max(1,N)   */
#define GEMM_F32_NULL_PTR 3      /* a needed matrix pointer is NULL         */
#define GEMM_F32_BAD_VARIANT 4   /* unknown variant                         */
#define GEMM_F32_LAUNCH_FAILED 5 /* the HIP runtime rejected the launch     */
#define GEMM_F32_MISALIGNED 6    /* a pointer is not 4-byte aligned         */
#define GEMM_F32_BAD_CONFIG 7    /* config outside the launch table, or not
                                    valid for this shape (small-K entries
                                    need K <= their BK)                      */
#define GEMM_F32_BAD_ARG 8       /* other invalid argument (query helpers)  */
#define GEMM_F32_BAD_WORKSPACE 9 /* split-K workspace NULL, too small or not
                                    4-byte aligned                          */
#define GEMM_F32_SCRATCH_TOO_SMALL 10 /* the plan's slabs exceed the fixed
                                         scratch of gemm_f32_splitk_noalloc */

/* ---- variants: the kernel ladder ------------------------------------ */
/* One thread per output element, operands read straight from global
 * memory, fp32 register accumulator (geek-doc.cn section 一; csh0101.cc
 * section "naive kernel 怎么读数据").  Workgroup 64 x 4 threads: one wave
 * covers 64 consecutive columns of one row. */
#define GEMM_F32_NAIVE 0
/* Textbook T x T tiled kernel with T = 16: per k step every thread loads one
 * A and one B element into LDS, barrier, T multiply-adds from LDS, barrier
 * (geek-doc.cn section 四; csh0101.cc section "代码里的样子"; ijyty.com steps
 * ①-⑧; mayulu.co section 6).  Elements outside the matrices are loaded as 0
 * (geek-doc.cn section 六; mayulu.co section 7). */
#define GEMM_F32_TILED 1
/* Production rung: fp32 matrix-core kernels (v_mfma_f32_16x16x4_f32, or
 * 32x32x2 in the register-staged entries), chosen per shape from a launch
 * table (gemm_f32_ex selects an entry, gemm_f32_tile reports the choice).
 * The default for large products is a persistent grid, one 256-thread
 * workgroup per CU, walking 256 x 256 output tiles in an XCD-aware order;
 * each of the 4 waves keeps a 128 x 128 block in accumulation registers (64
 * independent 16 x 16 MFMA chains); A and B go straight from global memory
 * into the idle one of two LDS stages (16-byte direct loads, chunks
 * permuted per row so fragment reads are free of bank conflicts), one
 * barrier per 32-deep k step; a partial last k step is filled through
 * registers with zeros past K; edge tiles are moved back inside C, and thin
 * remainder strips run on their own kernel, which also computes whole
 * products of at most 32 rows (a stream of B, read once);
 * products of at most 16 columns run on a thin-N kernel (a stream of A).
 * Few-tile products split each tile's k steps over the 4 waves and add the
 * partial tiles in wave order; K = 64 products keep A in LDS and stream B.
 * The "one thread, several outputs" and "register / wave / instruction
 * block" pyramid the pages point to (geek-doc.cn sections 三 and 五) on
 * CDNA4 matrix cores. */
#define GEMM_F32_PROD 2
/* The textbook kernel with T = 32 (1024 threads per workgroup). */
#define GEMM_F32_TILED32 3
/* The textbook kernel with T = 4, the pages' worked tile size (csh0101.cc
 * T = 4 example; ijyty.com 8x8 / TILE_SIZE = 4 example).  For tests and
 * teaching; slow. */
#define GEMM_F32_TILED4 4
/* The T = 32 textbook kernel with each LDS row padded by one float, the
 * shared-memory bank-conflict remedy the pages point to (geek-doc.cn
 * section 五).  Same results as GEMM_F32_TILED32; a measurement rung. */
#define GEMM_F32_TILED32_PAD 5
/* Register-blocked kernel on the vector ALU (no matrix cores): 128 x 128
 * workgroup tiles, 256 threads, each thread owns 8 x 8 outputs (four 4 x 4
 * blocks) in registers and does 64 fp32 FMAs per k from 16 LDS values; A is
 * stored k-major in LDS, two LDS stages, one barrier per 8- or 16-deep k
 * step (launch-table entries 0-3 and 4-5; entry 5 by default), out-of-range
 * elements loaded as 0.  The "one thread, several outputs"
 * step the pages point to (geek-doc.cn sections 三 and 五) without MFMA. */
#define GEMM_F32_VALU 6
#define GEMM_F32_NUM_VARIANTS 7

/*
 * gemm_f32 -- C = A x B (overwrite), see the layout above.
 *   M, N, K        problem size, each >= 0.  M == 0 or N == 0: no-op.
 *                  K == 0: C is set to 0 (the empty sum).
 *   A, lda         M x K operand, lda >= max(1, K).  May be NULL if M*K == 0.
 *   B, ldb         K x N operand, ldb >= max(1, N).  May be NULL if K*N == 0.
 *   C, ldc         M x N result, ldc >= max(1, N).  May be NULL if M*N == 0.
 *   variant        one of GEMM_F32_* variants above.
 *   stream         hipStream_t (NULL = null stream).
 * Returns GEMM_F32_OK or an error code; on error nothing is launched.
 */
int gemm_f32(int M, int N, int K, const float *A, int lda, const float *B,
             int ldb, float *C, int ldc, int variant, void *stream);

/*
 * gemm_f32_ex -- gemm_f32 with an explicit launch-table entry.
 *   config  -1 picks the entry gemm_f32 would use for this shape; otherwise
 *           an index below gemm_f32_num_configs(variant).  Production
 *           entries whose kernel holds all of K in one LDS stage ("panel"
 *           entries, reported with BK = their K limit) accept K <= BK only;
 *           the thin-M strip entry (reported with BN = 16, BK = 1 and BM =
 *           the rows a workgroup holds for this M) accepts M <= 32 only, the
 *           thin-N entry (BM = 16, BK = 1, BN = the columns it holds for
 *           this N) N <= 16 only.
 *           Whatever the entry, a thin remainder strip of rows or columns
 *           (an overhanging tile at most 1/8 full) is computed by further
 *           launches on the same stream: rows on the thin-M strip kernel,
 *           columns with small tiles.
 * Same semantics and errors as gemm_f32, plus GEMM_F32_BAD_CONFIG.
 */
int gemm_f32_ex(int M, int N, int K, const float *A, int lda, const float *B,
                int ldb, float *C, int ldc, int variant, int config,
                void *stream);

/*
 * ---- split-K ---------------------------------------------------------------
 * The pages tie the choice of tile size to occupancy (geek-doc.cn "矩阵乘法
 * tiling", section 六: block size interacts with occupancy, bank conflicts
 * and register pressure; mayulu.co "CUDA 编程系列之三", section 7: on-chip
 * memory per block is taken from occupancy).  This entry extends that
 * trade-off to products with fewer output tiles than the GPU has compute
 * units: instead of shrinking the tile, K is cut into chunks of kc values.  Workgroup (tile, chunk) computes the production kernel's tile
 * over its chunk into slab `chunk` of a workspace; a second kernel on the
 * same stream sums the slabs in chunk order into C.  The result is
 * deterministic for a given plan; it re-associates the k sum differently
 * from gemm_f32, so on non-integer inputs the two differ by rounding.
 *
 * gemm_f32_splitk_plan -- the plan gemm_f32_splitk would use (host only).
 *   config  -1 = automatic (entry 23's 128x128x32 tiles, 64x64 for outputs
 *           below 128x128), or a production k-loop entry (small-K panel and
 *           non-temporal-store entries are refused with GEMM_F32_BAD_CONFIG).
 *   splits  0 = automatic: the count with the least modelled time, from the
 *           busiest CU's share of (tile, chunk) pairs and the slab traffic,
 *           with at least four k steps per chunk, against the plain
 *           product's modelled time; products with a tile for every CU, or
 *           with fewer than 32 k steps, are not split.
 *           Else the requested count, capped at one k step per chunk.
 *   Writes the entry, the chunks actually used (1 means a plain product;
 *   with config -1 it then runs the entry gemm_f32 would choose),
 *   kc, and the workspace bytes needed (splits * M * N * 4, or 0 for one
 *   chunk).  Any output pointer may be NULL.
 *
 * gemm_f32_splitk -- C = A x B through that plan.  Arguments as gemm_f32_ex,
 * plus a device workspace of workspace_bytes (4-byte aligned, not
 * overlapping A, B or C; may be NULL when the plan needs none).  The
 * workspace's contents are overwritten and need no initialisation.
 * Returns GEMM_F32_BAD_WORKSPACE when it is missing or too small.
 */
int gemm_f32_splitk_plan(int M, int N, int K, int config, int splits,
                         int *config_out, int *splits_out, int *kc_out,
                         long long *workspace_bytes);
int gemm_f32_splitk(int M, int N, int K, const float *A, int lda,
                    const float *B, int ldb, float *C, int ldc, int config,
                    int splits, void *workspace, long long workspace_bytes,
                    void *stream);

/*
 * gemm_f32_splitk_noalloc -- gemm_f32_splitk for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation): the slabs live in a fixed device array
 * inside the library, GEMM_F32_NOALLOC_SCRATCH_BYTES per GPU, held from the
 * first call on that GPU until the process ends.  The call allocates nothing
 * (no hipMalloc, no hipFree, no allocating library routine); the caller
 * still owns A, B and C.
 *   Arguments as gemm_f32_splitk without the workspace; the plan is
 *   gemm_f32_splitk_plan's for (M, N, K, config, splits), so the result is
 *   bit for bit gemm_f32_splitk's with the same plan.
 *   stream  hipStream_t of the current device (NULL = its null stream);
 *           a stream of another device gives GEMM_F32_BAD_ARG.
 * Returns GEMM_F32_SCRATCH_TOO_SMALL, before anything is launched, when the
 * plan's workspace_bytes exceed GEMM_F32_NOALLOC_SCRATCH_BYTES (ask for
 * fewer splits, or use gemm_f32_splitk with a workspace); otherwise the
 * codes of gemm_f32_splitk.  Every call on one GPU shares that GPU's array
 * and leaves the last call's slabs in it: calls whose executions overlap on
 * one GPU (different streams, or host threads without ordering) race and
 * give undefined results.  The first call on a GPU looks up the array's
 * device address (hipGetSymbolAddress) with that GPU current.
 */
#define GEMM_F32_NOALLOC_SCRATCH_BYTES (64LL << 20)
int gemm_f32_splitk_noalloc(int M, int N, int K, const float *A, int lda,
                            const float *B, int ldb, float *C, int ldc, int config,
                            int splits, void *stream);

/* Number of launch-table entries of a variant (0 for an unknown variant). */
int gemm_f32_num_configs(int variant);

/*
 * gemm_f32_tile -- the launch-table entry a call would use (host only, no GPU
 * access).  For config == -1 the shape-based choice is reported.  Writes the
 * workgroup tile BM x BN, its k step BK, threads per workgroup and the entry
 * index actually chosen.  Any output pointer may be NULL.  For the naive
 * variant BM x BN is the 4 x 64 block of outputs a workgroup covers and BK
 * is 1.  Returns GEMM_F32_OK, GEMM_F32_BAD_VARIANT, GEMM_F32_BAD_CONFIG or
 * GEMM_F32_INVALID_DIM.
 */
int gemm_f32_tile(int variant, int config, int M, int N, int K, int *BM,
                  int *BN, int *BK, int *threads, int *chosen_config);

/*
 * gemm_f32_last_error -- detail of the last GEMM_F32_LAUNCH_FAILED returned
 * on the calling thread: the HIP runtime's error name and message, or "" if
 * no launch has failed on this thread.  The string is thread-local and stays
 * valid until the next failing call on the same thread.
 */
const char *gemm_f32_last_error(void);

/* Static message for a status code (never NULL). */
const char *gemm_f32_status_string(int status);

/* Library version string, e.g. "gemm_f32 0.1.0 gfx950". */
const char *gemm_f32_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F32_H */
