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

/*
 * 2-D convolution, the "Convolution" row of the tiled-kernel table in "Tiling
 * Strategies", section 5 ("Tiling Beyond GEMM"): input patches and filter
 * weights are the operands, and every weight is used at every output position.
 * The pages give no formula; this is the usual deep-learning form
 * (cross-correlation, zero padding, stride, dilation), channels innermost:
 *   x[n][h][w][c]    (N x H x W x C input, NHWC)
 *   wt[k][r][s][c]   (K x R x S x C filters, KRSC)
 *   y[n][p][q][k]    (N x P x Q x K output, NHWC),
 *   P = (H + 2 pad_h - dil_h (R - 1) - 1) / stride_h + 1 (floor; 0 if negative),
 *   Q = (W + 2 pad_w - dil_w (S - 1) - 1) / stride_w + 1,
 *   y[n][p][q][k] = sum_{r<R} sum_{s<S} sum_{c<C}
 *       x[n][p stride_h - pad_h + r dil_h][q stride_w - pad_w + s dil_w][c] * wt[k][r][s][c],
 * an input position outside 0 <= h < H, 0 <= w < W reading as zero.  The terms
 * are added in the order r, s, c (each ascending) in FP64, exact products as
 * for the matrix product; yabs is the same sum of |x| |wt| (the scale of the
 * acceptance bound).  y and yabs hold N * P * Q * K doubles.  Returns 0, or -1
 * for a negative size or a non-positive stride or dilation.
 */
static int64_t conv_out_size(int64_t in, int64_t pad, int64_t f, int64_t stride, int64_t dil) {
    const int64_t span = in + 2 * pad - dil * (f - 1) - 1;
    return span < 0 ? 0 : span / stride + 1;
}

typedef struct {
    int64_t N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, P, Q;
} conv_shape;

/* Output (n, p, q, k): terms in the order r, s, c. */
static void conv_one(const conv_shape *g, const float *x, const float *wt, int64_t n, int64_t p,
                     int64_t q, int64_t k, double *out, double *outabs) {
    double acc = 0.0, accabs = 0.0;
    for (int64_t r = 0; r < g->R; ++r) {
        const int64_t h = p * g->stride_h - g->pad_h + r * g->dil_h;
        if (h < 0 || h >= g->H) continue;
        for (int64_t s = 0; s < g->S; ++s) {
            const int64_t w = q * g->stride_w - g->pad_w + s * g->dil_w;
            if (w < 0 || w >= g->W) continue;
            const float *const xp = x + ((n * g->H + h) * g->W + w) * g->C;
            const float *const wp = wt + ((k * g->R + r) * g->S + s) * g->C;
            for (int64_t c = 0; c < g->C; ++c) {
                const double prod = (double)xp[c] * (double)wp[c];
                acc += prod;
                accabs += fabs(prod);
            }
        }
    }
    *out = acc;
    *outabs = accabs;
}

static int conv_setup(conv_shape *g, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                      int64_t R, int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                      int64_t stride_w, int64_t dil_h, int64_t dil_w) {
    if (N < 0 || H < 0 || W < 0 || C < 0 || K < 0 || R < 0 || S < 0 || pad_h < 0 || pad_w < 0)
        return -1;
    if (stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1) return -1;
    g->N = N; g->H = H; g->W = W; g->C = C; g->K = K; g->R = R; g->S = S;
    g->pad_h = pad_h; g->pad_w = pad_w; g->stride_h = stride_h; g->stride_w = stride_w;
    g->dil_h = dil_h; g->dil_w = dil_w;
    g->P = conv_out_size(H, pad_h, R, stride_h, dil_h);
    g->Q = conv_out_size(W, pad_w, S, stride_w, dil_w);
    return 0;
}

int oracle_conv2d_nhwc_f64(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R,
                           int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                           int64_t stride_w, int64_t dil_h, int64_t dil_w, const float *x,
                           const float *wt, double *y, double *yabs) {
    conv_shape g;
    if (conv_setup(&g, N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w))
        return -1;
    const int64_t outs = N * g.P * g.Q * K;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t e = 0; e < outs; ++e) {
        int64_t t = e;
        const int64_t k = t % K;
        t /= K;
        const int64_t q = t % g.Q;
        t /= g.Q;
        const int64_t p = t % g.P;
        conv_one(&g, x, wt, t / g.P, p, q, k, y + e, yabs + e);
    }
    return 0;
}

/* Selected outputs of the convolution above: flat output indices idx[e] into
 * the N x P x Q x K array; y[e], yabs[e] as there.  Returns 0 or -1. */
int oracle_conv2d_nhwc_entries_f64(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                                   int64_t R, int64_t S, int64_t pad_h, int64_t pad_w,
                                   int64_t stride_h, int64_t stride_w, int64_t dil_h,
                                   int64_t dil_w, const float *x, const float *wt, int64_t count,
                                   const int64_t *idx, double *y, double *yabs) {
    conv_shape g;
    if (conv_setup(&g, N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w))
        return -1;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t e = 0; e < count; ++e) {
        int64_t t = idx[e];
        const int64_t k = t % K;
        t /= K;
        const int64_t q = t % g.Q;
        t /= g.Q;
        const int64_t p = t % g.P;
        conv_one(&g, x, wt, t / g.P, p, q, k, y + e, yabs + e);
    }
    return 0;
}

/*
 * Attention, the "FlashAttention" row of the tiled-kernel table in "Tiling
 * Strategies", section 5 (tiled: Q, K and V blocks along the sequence;
 * reused: K and V blocks across query rows).  The pages give the tiling, not
 * the formula; this is scaled dot-product attention, one head at a time:
 *   Q[h][i][d] (Sq x D), K[h][j][d], V[h][j][d] (Skv x D), O[h][i][d] (Sq x D),
 *   s_ij = scale * sum_d Q[h][i][d] K[h][j][d],   j allowed when j < Skv and,
 *          if causal, j <= i,
 *   p_ij = exp(s_ij - max_j s_ij) over the allowed j,
 *   O[h][i][d] = sum_j p_ij V[h][j][d] / sum_j p_ij,
 * all in FP64 (the tiled, online-softmax form computes the same quantity).
 * A row with no allowed key (Skv = 0) is all zeros.  Also returned, per
 * output, mag = sum_j p_ij |V[h][j][d]| / sum_j p_ij (the scale of the
 * acceptance bound), and per row smax = max over allowed j of
 * scale * sum_d |Q[h][i][d]| |K[h][j][d]| (the size of the scores' rounding).
 * O and mag hold H*Sq*D doubles, smax H*Sq (mag and smax may be NULL).
 * Returns 0, or -1 for negative sizes.
 */
static void attention_row(int64_t Skv, int64_t D, double scale, int causal, int64_t i,
                          const float *q, const float *K, const float *V, double *s,
                          double *o, double *mag, double *smax) {
    const int64_t nj = causal ? (i + 1 < Skv ? i + 1 : Skv) : Skv;
    double m = -INFINITY, sm = 0.0;
    for (int64_t j = 0; j < nj; ++j) {
        double dot = 0.0, dabs = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            dot += (double)q[d] * (double)K[j * D + d];
            dabs += fabs((double)q[d] * (double)K[j * D + d]);
        }
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
        if (fabs(scale) * dabs > sm) sm = fabs(scale) * dabs;
    }
    double l = 0.0;
    for (int64_t j = 0; j < nj; ++j) {
        s[j] = exp(s[j] - m);  /* p_ij */
        l += s[j];
    }
    for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0, accabs = 0.0;
        for (int64_t j = 0; j < nj; ++j) {
            acc += s[j] * (double)V[j * D + d];
            accabs += s[j] * fabs((double)V[j * D + d]);
        }
        o[d] = nj > 0 ? acc / l : 0.0;
        if (mag) mag[d] = nj > 0 ? accabs / l : 0.0;
    }
    if (smax) *smax = sm;
}

int oracle_attention_f64(int64_t H, int64_t Sq, int64_t Skv, int64_t D, const float *Q,
                         const float *K, const float *V, float scale, int causal, double *O,
                         double *mag, double *smax) {
    if (H < 0 || Sq < 0 || Skv < 0 || D < 0) return -1;
#ifdef _OPENMP
#pragma omp parallel
#endif
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
#ifdef _OPENMP
#pragma omp for collapse(2) schedule(static)
#endif
        for (int64_t h = 0; h < H; ++h) {
            for (int64_t i = 0; i < Sq; ++i) {
                const int64_t row = h * Sq + i;
                attention_row(Skv, D, (double)scale, causal, i, Q + row * D, K + h * Skv * D,
                              V + h * Skv * D, s, O + row * D, mag ? mag + row * D : NULL,
                              smax ? smax + row : NULL);
            }
        }
        free(s);
    }
    return 0;
}

/* Selected rows (h, i) of the attention above: rows[e] = h * Sq + i; O, mag
 * hold count * D doubles, smax count.  Returns 0 or -1. */
int oracle_attention_rows_f64(int64_t H, int64_t Sq, int64_t Skv, int64_t D, const float *Q,
                              const float *K, const float *V, float scale, int causal,
                              int64_t count, const int64_t *rows, double *O, double *mag,
                              double *smax) {
    if (H < 0 || Sq < 0 || Skv < 0 || D < 0) return -1;
#ifdef _OPENMP
#pragma omp parallel
#endif
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t e = 0; e < count; ++e) {
            const int64_t h = rows[e] / (Sq > 0 ? Sq : 1);
            const int64_t i = rows[e] - h * Sq;
            attention_row(Skv, D, (double)scale, causal, i, Q + rows[e] * D, K + h * Skv * D,
                          V + h * Skv * D, s, O + e * D, mag + e * D, smax + e);
        }
        free(s);
    }
    return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
