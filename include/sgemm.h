/*
 * sgemm.h -- C ABI of the MI355X (gfx950) FP32 matrix-multiply library.
 *
 * Operation (every entry point below computes it):
 *   C[i*ldc + j] = sum_{k<K} A[i*lda + k] * B[k*ldb + j]     for i < M, j < N,
 * i.e. C = A x B with A (M x K), B (K x N) and C (M x N) row-major, each row
 * starting a leading dimension after the previous one.  This is the product
 * defined in "Tiling Hierarchy on GPUs" (introduction and section "Inner
 * Product": each output is a K-term sum of products) and in "Tiling
 * Strategies" section 2 ("The Problem").  As in "CMU DLSys Lecture 12: GPU
 * Acceleration" section 5, the accumulators start at zero and C is never read:
 * C's M x N window is overwritten (beta = 0), and nothing outside that window
 * (the ldc padding, other memory) is written.  Padding between a row's end and
 * its leading dimension is never read.  The order in which the K products of
 * one element are summed is unspecified; results are IEEE FP32 with
 * round-to-nearest-even; integer-valued inputs whose partial sums stay below
 * 2^24 give the exact integer result.
 *
 * Memory and ownership: A, B and C are device pointers owned by the caller.
 * The library never allocates, frees or copies memory between host and
 * device, and keeps no mutable global state, so calls from several host
 * threads are safe.  C must not overlap A or B (not checked).
 *
 * Asynchrony: work is enqueued on `stream` (NULL is the default stream) and
 * the call returns without waiting for it ("CMU DLSys Lecture 12" section 2:
 * launches are asynchronous and completion follows the stream's rules).  The
 * caller synchronises before reading C.
 *
 * Errors: every entry point returns an sgemm_status_t.  Argument errors are
 * detected on the host before anything is enqueued; a launch error reported
 * by HIP is returned as SGEMM_STATUS_LAUNCH_FAILED.
 *
 * Degenerate sizes: M == 0, N == 0 or batch == 0 is a successful no-op.
 * K == 0 with M, N > 0 writes +0.0 to C's M x N window (the empty sum).
 */
#ifndef TILED_FP32_SGEMM_H
#define TILED_FP32_SGEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sgemm_status {
    SGEMM_STATUS_SUCCESS = 0,
    /* M, N, K or batch is negative. */
    SGEMM_STATUS_INVALID_SIZE = -1,
    /* lda < max(1, K), ldb < max(1, N) or ldc < max(1, N). */
    SGEMM_STATUS_INVALID_LD = -2,
    /* A, B or C is NULL although the call would read or write it. */
    SGEMM_STATUS_NULL_POINTER = -3,
    /* M, N, K or batch is 2^31 or more, an element offset overflows 64 bits, or
       one product's tile grid needs more than 2^32 - 1 work-items (a single
       launch's limit; a batch is split over as many launches as it needs). */
    SGEMM_STATUS_SIZE_OVERFLOW = -4,
    /* A batch stride is negative, or strideC lets two C matrices overlap. */
    SGEMM_STATUS_INVALID_STRIDE = -5,
    /* HIP reported an error when the kernel was enqueued. */
    SGEMM_STATUS_LAUNCH_FAILED = -6,
    /* The tile configuration index is unknown, or (general form) the tile is
       not built for the general form. */
    SGEMM_STATUS_INVALID_CONFIG = -7,
    /* A transpose flag of the general form is neither 0 nor 1. */
    SGEMM_STATUS_INVALID_OP = -8,
    /* Split-K: the workspace is NULL or smaller than sgemm_splitk_plan
       reports for the same arguments. */
    SGEMM_STATUS_INVALID_WORKSPACE = -9,
    /* sgemm_splitk_noalloc: the requested tile and chunk count need more
       workspace than SGEMM_SPLITK_SCRATCH_BYTES. */
    SGEMM_STATUS_SCRATCH_TOO_SMALL = -10
} sgemm_status_t;

/*
 * Single product on the matrix cores (v_mfma_f32_32x32x2_f32, or
 * v_mfma_f32_16x16x4_f32 on the 96 x 96 tile), block tile chosen from the
 * shape.  Arguments: sizes M, N, K (>= 0); A with leading
 * dimension lda; B with ldb; C with ldc; stream.
 */
int sgemm(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
          int64_t ldb, float *C, int64_t ldc, hipStream_t stream);

/*
 * `batch` independent products.  Product b reads A + b*strideA and
 * B + b*strideB and writes C + b*strideC (strides in elements, >= 0).
 * strideA or strideB may be 0 (a shared operand); for batch > 1, strideC must
 * be at least (M-1)*ldc + N so that the C matrices do not overlap.
 */
int sgemm_strided_batched(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                          int64_t strideA, const float *B, int64_t ldb, int64_t strideB,
                          float *C, int64_t ldc, int64_t strideC, int64_t batch,
                          hipStream_t stream);

/*
 * The same two operations on the vector ALUs: each lane owns an 8x8 register
 * tile of a 128x128 block tile and updates it with FP32 fused multiply-adds,
 * the thread-tile design of "Tiling Hierarchy on GPUs" (sections "Register
 * Tiling" and "Register prefetching") and "Tiling Strategies" section 4
 * ("Register Tiling").  Same contract as sgemm / sgemm_strided_batched.
 */
int sgemm_valu(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
               int64_t ldb, float *C, int64_t ldc, hipStream_t stream);

int sgemm_valu_strided_batched(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                               int64_t strideA, const float *B, int64_t ldb, int64_t strideB,
                               float *C, int64_t ldc, int64_t strideC, int64_t batch,
                               hipStream_t stream);

/*
 * General form C = alpha * op(A) * op(B) + beta * C on the matrix cores,
 * row-major like the plain product.  C is M x N (ldc >= max(1, N)).
 *   transA = 0: A is stored M x K (lda >= max(1, K)), op(A) = A.
 *   transA = 1: A is stored K x M (lda >= max(1, M)), op(A) = A^T; this is
 *     the form "CMU DLSys Lecture 12: GPU Acceleration" section 4 writes the
 *     product in, C = A^T B.
 *   transB = 0: B is stored K x N (ldb >= max(1, N)); transB = 1: B is stored
 *     N x K (ldb >= max(1, K)), op(B) = B^T.
 * alpha and beta follow the BLAS convention (the pages have neither; their
 * product is alpha = 1, beta = 0): beta == 0 means C is not read, so it may
 * hold anything, NaN included; alpha == 0 or K == 0 means there is no product
 * term, A and B are not read (and may be NULL), and C becomes beta * C (+0
 * when beta == 0; nothing is enqueued when beta == 1).  Other flag values
 * give SGEMM_STATUS_INVALID_OP.  Errors, ownership and stream behaviour as
 * for sgemm; the operands are read in place, whatever their layout (each
 * stored layout has its own global->LDS copy, nothing is transposed in
 * memory).
 */
int sgemm_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
             const float *A, int64_t lda, const float *B, int64_t ldb, float beta, float *C,
             int64_t ldc, hipStream_t stream);

/* Strided batch of the general form; strides as for sgemm_strided_batched. */
int sgemm_ex_strided_batched(int transA, int transB, int64_t M, int64_t N, int64_t K,
                             float alpha, const float *A, int64_t lda, int64_t strideA,
                             const float *B, int64_t ldb, int64_t strideB, float beta, float *C,
                             int64_t ldc, int64_t strideC, int64_t batch, hipStream_t stream);

/*
 * The general form with an explicit tile configuration, for tests and
 * tuning; SGEMM_STATUS_INVALID_CONFIG if the index is unknown or the tile is
 * not built for the general form (sgemm_config_has_general_form).
 */
int sgemm_ex_with_config(int config, int transA, int transB, int64_t M, int64_t N, int64_t K,
                         float alpha, const float *A, int64_t lda, int64_t strideA,
                         const float *B, int64_t ldb, int64_t strideB, float beta, float *C,
                         int64_t ldc, int64_t strideC, int64_t batch, hipStream_t stream);

/* 1 if tile configuration `config` is built for the general form (all four
   layouts), 0 if not, SGEMM_STATUS_INVALID_CONFIG if unknown.  Host only. */
int sgemm_config_has_general_form(int config);

/* The configuration sgemm_ex would use for this shape (any layout).  Host
   only; a negative status for bad sizes. */
int sgemm_select_general_config(int64_t M, int64_t N, int64_t K, int64_t batch);

/*
 * Matrix-core product with an explicit block-tile configuration, for tests
 * and tuning ("Tiling Strategies" section 4: tile size trades reuse against
 * occupancy and tail effects; "Tiling Hierarchy on GPUs", "Reducing Overhead
 * Slots": libraries tune the tile per shape).  `config` is an index below
 * sgemm_num_configs(); otherwise SGEMM_STATUS_INVALID_CONFIG.  batch == 1 with
 * zero strides is a single product.
 */
int sgemm_with_config(int config, int64_t M, int64_t N, int64_t K, const float *A,
                      int64_t lda, int64_t strideA, const float *B, int64_t ldb,
                      int64_t strideB, float *C, int64_t ldc, int64_t strideC, int64_t batch,
                      hipStream_t stream);

/* Number of matrix-core tile configurations. */
int sgemm_num_configs(void);

/*
 * Description of configuration `config` written into `buf` (at most `len`
 * bytes, NUL-terminated), e.g. "mfma_256x128x16_w2x2".  Returns 0, or
 * SGEMM_STATUS_INVALID_CONFIG.  Also fills the block-tile sizes when the
 * pointers are not NULL.  Host only; touches no device.
 */
int sgemm_config_info(int config, char *buf, int64_t len, int *bm, int *bn, int *bk,
                      int *threads);

/*
 * The configuration sgemm / sgemm_strided_batched would use for this shape:
 * the one with the smallest predicted time (sgemm_config_predict_us).  Host
 * only; touches no device.  Returns a negative status for bad sizes.
 */
int sgemm_select_config(int64_t M, int64_t N, int64_t K, int64_t batch);

/*
 * 1 if the automatic choice may pick configuration `config`, 0 if it is a
 * control build kept for measurements only, SGEMM_STATUS_INVALID_CONFIG for
 * an unknown index.  Host only.
 */
int sgemm_config_selectable(int config);

/*
 * Workgroups of configuration `config` one compute unit can hold at once:
 * the HIP runtime's occupancy answer for the kernel (registers as compiled,
 * LDS), or, when no device is available, the floor the tile's launch bound
 * and LDS footprint guarantee.  Host only; SGEMM_STATUS_INVALID_CONFIG for an
 * unknown index.
 */
int sgemm_config_workgroups_per_cu(int config);

/*
 * Predicted microseconds of one launch of configuration `config` on this
 * shape, from a per-configuration time model fitted to measurements (the
 * tile-size trade-off of "Tiling Strategies" section 4, in numbers): whole
 * rounds of 256 * w tiles, where w workgroups overlap on a CU, each costing
 * BM*BN*(a + b*K), and a partial last round in proportion.  A negative value
 * is a status code (unknown or control configuration, bad sizes).  Host
 * only.
 */
double sgemm_config_predict_us(int config, int64_t M, int64_t N, int64_t K, int64_t batch);

/*
 * Measure instead of predicting: times every selectable configuration on the
 * caller's operands (one warm-up launch, then `reps` launches between two
 * events on `stream`), stores the fastest in *best_config and its mean
 * milliseconds per launch in *best_ms (if not NULL), and finally runs the
 * fastest once more, so that C holds A x B on return.  Arguments are checked
 * as for sgemm_strided_batched (plus best_config != NULL and reps >= 1);
 * empty products and K = 0 return the automatic choice without timing.  This
 * call blocks the host until the timed work on `stream` is done and creates
 * two HIP events; it allocates no device memory.  Returns 0 or a negative
 * status (the first failing launch's).
 */
int sgemm_autotune(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                   int64_t strideA, const float *B, int64_t ldb, int64_t strideB, float *C,
                   int64_t ldc, int64_t strideC, int64_t batch, hipStream_t stream, int reps,
                   int *best_config, float *best_ms);

/*
 * Split-K product for under-filled grids, C = A x B with the semantics of
 * sgemm (row-major, beta = 0, C's window overwritten and nothing else
 * written).  The k loop of "Tiling Strategies" section 2 is cut into `splits`
 * chunks of whole BK slices; each output tile gets one workgroup per chunk,
 * so a thin product (few BM x BN tiles, long K) still fills the CUs.  The
 * chunks' partial tiles join inside the same launch: each workgroup writes
 * its partial to the workspace and counts itself in on the tile's counter;
 * the last one to arrive adds the partials in chunk order 0, 1, ... (so the
 * result does not depend on timing and is bit-reproducible), resets the
 * counter and stores the tile.  No workgroup waits for another.  With
 * splits = 0 the plan may be hybrid: when the tile count is not a multiple of
 * the 256 CUs, the tiles of the whole layers (one tile per CU each) take all
 * of K and only the R tiles of the last partial layer are split, so that
 * their chunks even out the work per CU ("Tiling Strategies" section 4 on
 * tail effects; sgemm_splitk_plan_full_tiles reports the unsplit tiles).
 *
 * config: a configuration with a split-K variant (sgemm_config_has_splitk),
 *   or -1 for the choice of the time model (which may be the plain kernel).
 * splits: requested chunk count, 1 ... 64, or 0 for the time model's choice;
 *   the count used is at most ceil(K / BK) (sgemm_splitk_plan reports it).
 * workspace, workspace_bytes: device memory owned by the caller, at least
 *   sgemm_splitk_plan(...) bytes for the same config, sizes and splits
 *   (a count that resolves to one chunk needs none: NULL and 0 are accepted).
 *   Layout: its first SGEMM_SPLITK_HEADER_BYTES hold one uint32 arrival
 *   counter per output tile (tile t's at word t, for every shape), the
 *   partial tiles follow.  The header must hold zeros before the first use
 *   (e.g. allocated with hipMemset or torch.zeros); every call that completes
 *   leaves it zero again, so one workspace is zeroed once and then serves
 *   calls of any shape and chunk count in turn.  Calls that may run at the
 *   same time need workspaces of their own; concurrent calls on one
 *   workspace race.  A product with more than SGEMM_SPLITK_MAX_TILES output
 *   tiles is not split (the plan reports one chunk).
 * Errors as for sgemm, plus SGEMM_STATUS_INVALID_CONFIG (no split-K variant),
 * SGEMM_STATUS_INVALID_SIZE (splits outside 0 ... 64) and
 * SGEMM_STATUS_INVALID_WORKSPACE; on an error nothing is enqueued.
 */
#define SGEMM_SPLITK_MAX_TILES 16384
#define SGEMM_SPLITK_HEADER_BYTES (SGEMM_SPLITK_MAX_TILES * 4)
int sgemm_splitk(int config, int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                 const float *B, int64_t ldb, float *C, int64_t ldc, int64_t splits,
                 void *workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * sgemm_splitk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same product, kernels and chunk-order join, with the workspace taken
 * from a buffer the library holds, SGEMM_SPLITK_SCRATCH_BYTES (64 MiB) per
 * GPU, kept from the first call on that GPU until the process ends.  The
 * caller passes only inputs, output and stream; the call allocates and frees
 * nothing.  Its first call on a GPU looks up that GPU's buffer and enqueues
 * one small kernel that zeroes the counter header (again on later calls
 * until one such launch was made outside graph capture); every completed
 * call leaves the header zero.
 *
 * config, splits: as for sgemm_splitk.  With config = -1 and splits = 0 the
 * time model chooses among the plans whose workspace fits the buffer (the
 * plain kernel always does); an explicit tile or chunk count whose plan
 * needs more returns SGEMM_STATUS_SCRATCH_TOO_SMALL.  Results are bit for
 * bit those of sgemm_splitk with the same plan.
 * Every call on one GPU shares that GPU's buffer: calls that may overlap on
 * one GPU (other streams, other host threads) race and must use
 * sgemm_splitk with workspaces of their own.
 * Errors as for sgemm_splitk, plus SGEMM_STATUS_SCRATCH_TOO_SMALL, and
 * SGEMM_STATUS_LAUNCH_FAILED when HIP cannot name the stream's device or the
 * buffer's address; on an error nothing is enqueued.
 */
#define SGEMM_SPLITK_SCRATCH_BYTES (64 * 1024 * 1024)
int sgemm_splitk_noalloc(int config, int64_t M, int64_t N, int64_t K, const float *A,
                         int64_t lda, const float *B, int64_t ldb, float *C, int64_t ldc,
                         int64_t splits, hipStream_t stream);

/*
 * The plan sgemm_splitk would run for these arguments: stores the tile
 * configuration in *plan_config and the chunk count in *plan_splits (either
 * pointer may be NULL) and returns the workspace bytes it needs (0 for one
 * chunk or an empty product), or a negative status.  Host only.
 */
int64_t sgemm_splitk_plan(int config, int64_t M, int64_t N, int64_t K, int64_t splits,
                          int *plan_config, int64_t *plan_splits);

/*
 * For the plan sgemm_splitk would run with these arguments: the number of
 * output tiles that take all of K without a join (0 when every tile is split
 * or the plan is the plain kernel), or a negative status.  Host only.
 */
int64_t sgemm_splitk_plan_full_tiles(int config, int64_t M, int64_t N, int64_t K,
                                     int64_t splits);

/* 1 if configuration `config` has a split-K variant, 0 if not,
   SGEMM_STATUS_INVALID_CONFIG if unknown.  Host only. */
int sgemm_config_has_splitk(int config);

/*
 * The general form C = alpha op(A) op(B) + beta C (as sgemm_ex, one product)
 * with its reduction split as in sgemm_splitk: chunk b of every output tile
 * reduces k in [b kchunk, (b+1) kchunk) over the stored layouts, the chunks
 * join in chunk order through the caller's workspace, and the joining
 * workgroup stores alpha times the sum, plus beta C when beta != 0 (C is
 * read once, by that store).  For thin products with a long K, where one
 * tile per CU leaves most of the machine idle ("Tiling Strategies" section 4
 * on tile size and tail effects; "CMU DLSys Lecture 12: GPU Acceleration" section 4 writes the
 * product as C = A^T B with A stored K x M, the transA = 1 layout here).
 *
 * transA, transB, sizes, scalars, A, lda, B, ldb, C, ldc: as for sgemm_ex.
 * config: a configuration with general-form split-K variants
 *   (sgemm_config_has_general_splitk), or -1 for the time model's choice,
 *   which may be the unsplit general form.
 * splits, workspace, workspace_bytes: as for sgemm_splitk, with the size
 *   sgemm_ex_splitk_plan reports; the same workspace layout, header and
 *   zero-once rule, so one workspace serves sgemm_splitk and this call in
 *   turn.  alpha = 0 or K = 0 scale C by beta and use no workspace.
 * Results are bit for bit those of the same plan's chunks summed in chunk
 * order, independent of timing.  Errors as for sgemm_ex and sgemm_splitk; on
 * an error nothing is enqueued.
 */
int sgemm_ex_splitk(int config, int transA, int transB, int64_t M, int64_t N, int64_t K,
                    float alpha, const float *A, int64_t lda, const float *B, int64_t ldb,
                    float beta, float *C, int64_t ldc, int64_t splits, void *workspace,
                    int64_t workspace_bytes, hipStream_t stream);

/*
 * The plan sgemm_ex_splitk would run with these arguments: its tile in
 * *plan_config and chunk count in *plan_splits (either pointer may be NULL),
 * and the workspace bytes it needs as the return value (0 when it runs one
 * chunk or the product is empty), or a negative status.  Host only.
 */
int64_t sgemm_ex_splitk_plan(int config, int transA, int transB, int64_t M, int64_t N,
                             int64_t K, int64_t splits, int *plan_config, int64_t *plan_splits);

/*
 * For the plan sgemm_ex_splitk would run with these arguments: the number of
 * output tiles that take all of K without a join (0 when every tile is split
 * or the plan is unsplit), or a negative status.  Host only.
 */
int64_t sgemm_ex_splitk_plan_full_tiles(int config, int transA, int transB, int64_t M,
                                        int64_t N, int64_t K, int64_t splits);

/* 1 if configuration `config` has split-K variants of the general form (all
   four layouts), 0 if not, SGEMM_STATUS_INVALID_CONFIG if unknown.  Host
   only. */
int sgemm_config_has_general_splitk(int config);

/* Static text for a status code (never NULL). */
const char *sgemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TILED_FP32_SGEMM_H */
