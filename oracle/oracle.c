/*
 * CPU oracle for the FP32 matrix product C = A x B (row-major, leading dimensions).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the GPU path may include, link or call
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (plain definition, no tiling):
 *   "Tiling Hierarchy on GPUs", section "Inner Product": each output element is
 *   the K-term sum C[i][j] = sum_k A[i][k] * B[k][j]; the whole product is
 *   M*N*K fused multiply-adds.  "Tiling Strategies", section 2 "The Problem",
 *   prints the same loop over k for one C[i][j].
 *   "CMU DLSys Lecture 12: GPU Acceleration", section 5: accumulators start at
 *   zero and C is never read, so this is the beta = 0 product.
 *
 * Precision: every FP32 x FP32 product is exact in FP64 (24 + 24 significand
 * bits <= 53), and the K-term FP64 running sum has relative error at most
 * about K * 2^-53 of sum_k |A[i][k]| |B[k][j]|, so the result is the exact
 * product to within far less than one FP32 ulp for the sizes used here.
 * Alongside C it returns Cabs[i][j] = sum_k |A[i][k]| |B[k][j]|, the scale the
 * acceptance bound |C_gpu - C| <= 2e-4 * Cabs is written against.
 *
 * Order: for every (i, j) the terms are added for k = 0, 1, ..., K-1 in that
 * order, whatever the thread count, so results do not depend on threading.
 * Rows are split over OpenMP threads; that reorders no sum.
 *
 * Padding between the end of a row and its leading dimension is never read.
 * K = 0 gives exact zeros (the empty sum).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One row i of C: acc[j] and accabs[j] over j < N, k ascending. */
static void row_product(int64_t N, int64_t K, const float *Arow, const float *B,
                        int64_t ldb, double *acc, double *accabs) {
    for (int64_t j = 0; j < N; ++j) {
        acc[j] = 0.0;
        accabs[j] = 0.0;
    }
    for (int64_t k = 0; k < K; ++k) {
        const double a = (double)Arow[k];
        const double aa = fabs(a);
        const float *Bk = B + k * ldb;
        for (int64_t j = 0; j < N; ++j) {
            const double b = (double)Bk[j];
            acc[j] += a * b;
            accabs[j] += aa * fabs(b);
        }
    }
}

/*
 * Full product.  C and Cabs are M x N row-major FP64 with leading dimension ldc
 * (Cabs may be NULL).  nthreads <= 0 means "all available".
 * Returns the number of threads used.
 */
int oracle_sgemm_f64(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                     const float *B, int64_t ldb, double *C, double *Cabs, int64_t ldc,
                     int nthreads) {
    int used = 1;
    if (M <= 0 || N <= 0) return used;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    if (nthreads > M) nthreads = (int)M;
    used = nthreads;
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *scratch_abs = NULL;
        if (Cabs == NULL) scratch_abs = (double *)malloc(sizeof(double) * (size_t)N);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t i = 0; i < M; ++i) {
            double *abs_row = Cabs ? Cabs + i * ldc : scratch_abs;
            row_product(N, K, A + i * lda, B, ldb, C + i * ldc, abs_row);
        }
        free(scratch_abs);
    }
    return used;
}

/*
 * Strided batch: for b < batch, matrix b of each operand starts at
 * b * stride{A,B} floats; C and Cabs (M x N each, leading dimension ldc)
 * are written at b * strideC doubles.
 */
int oracle_sgemm_strided_batched_f64(int64_t M, int64_t N, int64_t K, const float *A,
                                     int64_t lda, int64_t strideA, const float *B,
                                     int64_t ldb, int64_t strideB, double *C, double *Cabs,
                                     int64_t ldc, int64_t strideC, int64_t batch,
                                     int nthreads) {
    int used = 1;
    for (int64_t b = 0; b < batch; ++b) {
        used = oracle_sgemm_f64(M, N, K, A + b * strideA, lda, B + b * strideB, ldb,
                                C + b * strideC, Cabs ? Cabs + b * strideC : NULL, ldc,
                                nthreads);
    }
    return used;
}

/*
 * Selected entries only: out[e] = sum_k A[rows[e]][k] * B[k][cols[e]] with the
 * same k-ascending FP64 sum as the full product, so each value is bitwise equal
 * to the corresponding entry of oracle_sgemm_f64.  Used where the full product
 * would take too long on the CPU.
 */
void oracle_sgemm_entries_f64(int64_t K, const float *A, int64_t lda, const float *B,
                              int64_t ldb, int64_t n_entries, const int64_t *rows,
                              const int64_t *cols, double *out, double *out_abs) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t e = 0; e < n_entries; ++e) {
        const float *Arow = A + rows[e] * lda;
        const float *Bcol = B + cols[e];
        double acc = 0.0, accabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)Arow[k];
            const double b = (double)Bcol[k * ldb];
            acc += a * b;
            accabs += fabs(a) * fabs(b);
        }
        out[e] = acc;
        if (out_abs) out_abs[e] = accabs;
    }
}

/*
 * General form C = alpha * op(A) op(B) + beta * C, row-major.
 *
 * op(A) is the M x K matrix A (stored M x K, leading dimension lda) when
 * transA == 0, and the transpose of the stored K x M matrix when transA != 0:
 * op(A)[i][k] = A[k*lda + i].  "CMU DLSys Lecture 12: GPU Acceleration",
 * section 4, writes the product in exactly that form, C = A^T B with A stored
 * K x M.  op(B) is the K x N matrix B (stored K x N, ldb) when transB == 0,
 * else the transpose of the stored N x K matrix: op(B)[k][j] = B[j*ldb + k].
 *
 * alpha and beta are the usual scalar update; the pages have none (their
 * accumulators start at zero and C is not read, which is alpha = 1, beta = 0).
 * The reading taken is the standard BLAS one: with beta == 0, C_in is not
 * read at all (so NaN or garbage there does not matter); with alpha == 0 or
 * K == 0 there is no product term at all (A and B are not read), so the
 * result is beta * C_in, or +0 when beta == 0.
 *
 * Every element is the same k-ascending FP64 sum as oracle_sgemm_f64; then
 * out = alpha * sum + beta * C_in in FP64, and
 * out_abs = |alpha| * sum_k |op(A)[i][k]| |op(B)[k][j]| + |beta| * |C_in|,
 * the scale of the acceptance bound.  C_in (float, leading dimension ldc_in)
 * may be NULL when beta == 0; out and out_abs are M x N with leading
 * dimension ldo (out_abs may be NULL).
 */
static void element_ex(int transA, int transB, int64_t i, int64_t j, int64_t K, double alpha,
                       const float *A, int64_t lda, const float *B, int64_t ldb, double beta,
                       const float *C_in, int64_t ldc_in, double *out, double *out_abs) {
    const int has_product = alpha != 0.0 && K > 0;
    double v = 0.0, vabs = 0.0;
    if (has_product) {
        double acc = 0.0, accabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)(transA ? A[k * lda + i] : A[i * lda + k]);
            const double b = (double)(transB ? B[j * ldb + k] : B[k * ldb + j]);
            acc += a * b;
            accabs += fabs(a) * fabs(b);
        }
        v = alpha * acc;
        vabs = fabs(alpha) * accabs;
    }
    if (beta != 0.0) {
        const double c = (double)C_in[i * ldc_in + j];
        v = has_product ? v + beta * c : beta * c;
        vabs += fabs(beta) * fabs(c);
    }
    *out = v;
    if (out_abs) *out_abs = vabs;
}

int oracle_sgemm_ex_f64(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                        const float *A, int64_t lda, const float *B, int64_t ldb, float beta,
                        const float *C_in, int64_t ldc_in, double *out, double *out_abs,
                        int64_t ldo, int nthreads) {
    int used = 1;
    if (M <= 0 || N <= 0) return used;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    if (nthreads > M) nthreads = (int)M;
    used = nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            element_ex(transA, transB, i, j, K, (double)alpha, A, lda, B, ldb, (double)beta,
                       C_in, ldc_in, out + i * ldo + j, out_abs ? out_abs + i * ldo + j : NULL);
        }
    }
    return used;
}

/* Selected entries of the general form; bitwise equal to the full version. */
void oracle_sgemm_ex_entries_f64(int transA, int transB, int64_t K, float alpha,
                                 const float *A, int64_t lda, const float *B, int64_t ldb,
                                 float beta, const float *C_in, int64_t ldc_in,
                                 int64_t n_entries, const int64_t *rows, const int64_t *cols,
                                 double *out, double *out_abs) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t e = 0; e < n_entries; ++e) {
        element_ex(transA, transB, rows[e], cols[e], K, (double)alpha, A, lda, B, ldb,
                   (double)beta, C_in, ldc_in, out + e, out_abs ? out_abs + e : NULL);
    }
}

/*
 * Sliding window sums ("CMU DLSys Lecture 12: GPU Acceleration", section 3):
 * y[i] = sum_{d=0}^{W-1} x[i+d] for 0 <= i < n, where n counts outputs and the
 * input holds n + W - 1 valid elements (the lecture's five-wide case is
 * W = 5; its general width is W = 2R + 1, and any W >= 1 is read the same
 * way).  The terms are added for d = 0, 1, ..., W-1 in FP64 (exact for FP32
 * inputs up to W ~ 2^29), and yabs[i] = sum_d |x[i+d]| is the scale of the
 * acceptance bound.  yabs may be NULL.
 */
void oracle_window_sum_f64(int64_t n, int64_t W, const float *x, double *y, double *yabs) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0, sa = 0.0;
        for (int64_t d = 0; d < W; ++d) {
            const double v = (double)x[i + d];
            s += v;
            sa += fabs(v);
        }
        y[i] = s;
        if (yabs) yabs[i] = sa;
    }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
