/*
 * oracle_sgemm.c -- plain, slow, obviously correct CPU SGEMM in float64.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the GPU library is tested against,
 * not part of it: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may build, load or call it.  It shares no code, header or
 * table with the HIP library and includes nothing from it.
 *
 * What it computes (the plain definition, written out):
 *   "如何高效实现矩阵乘？CUDA初学者的角度入门", section "樸素 GEMM 與前置知識"
 *   (naive GEMM): A is an M x K row-major matrix, B is K x N row-major, C is
 *   M x N row-major, alpha and beta are scalars, and the kernel forms
 *   c = sum_k A[i][k] * B[k][j] and then stores C = beta*C + alpha*c, so alpha
 *   is applied once to the finished dot product.
 *
 *   For every (i, j):
 *     ref[i][j] = (double)alpha * S_ij + (double)beta * (double)C[i][j]
 *     S_ij      = sum_{k=0..K-1} (double)A[i][k] * (double)B[k][j]
 *   with the sum formed from 0.0 in ascending k.  The beta term is dropped
 *   when beta == 0 (BLAS convention: C is then not read, so NaN or Inf in C
 *   does not propagate), and the alpha term is dropped when alpha == 0 (the
 *   same convention for A and B: they are not read, so NaN or Inf in them
 *   does not propagate and ref = beta * C).  Element (r, c) of a matrix
 *   with leading dimension ld sits at r*ld + c.
 *
 *   Every product of two floats is exact in double (24 + 24 < 53 significand
 *   bits); only the sums and the two scalings round.
 *
 *   It also forms the error denominator of the pass rule in the same pass:
 *     den[i][j] = |alpha| * sum_k |A[i][k]| * |B[k][j]| + |beta| * |C[i][j]| + 1e-30
 *   (the |beta| term only when beta != 0).
 *
 * Entry points:
 *   oracle_sgemm_rows    rows [row0, row0+nrows) of ref and den, every column,
 *                        split over POSIX threads by row.  Each thread walks
 *                        i, then k, then j with two double row accumulators,
 *                        so each element's sum still starts at 0.0 and adds
 *                        its terms in ascending k: the same sums, bit for bit,
 *                        as the i-j-k loop of the points entry below.
 *   oracle_sgemm_points  ref and den at an explicit list of (row, col) pairs,
 *                        one dot product each, in the i-j-k form of the
 *                        definition.
 *   oracle_nthreads      the thread count that nthreads <= 0 resolves to.
 *
 * Return value: 0 on success, -1 on a bad argument (negative size, bad leading
 * dimension, NULL where data is needed, index out of range), -2 when a thread
 * or buffer cannot be created.  Outputs are left unspecified on error.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_DEN_FLOOR 1e-30

int oracle_nthreads(void)
{
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static int bad_args(int M, int N, int K, float alpha, const float *A, int lda,
                    const float *B, int ldb, float beta, const float *C,
                    int ldc)
{
    if (M < 0 || N < 0 || K < 0)
        return 1;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return 1;
    if (alpha != 0.0f && ((M > 0 && K > 0 && A == NULL) || (K > 0 && N > 0 && B == NULL)))
        return 1;
    if (beta != 0.0f && M > 0 && N > 0 && C == NULL)
        return 1;
    return 0;
}

struct band {
    int M, N, K;
    double alpha, beta;
    const float *A, *B, *C;
    int lda, ldb, ldc;
    int r_begin, r_end; /* absolute rows */
    int row0;           /* first row of the output band */
    double *ref, *den;
    int status;
};

static void *run_band(void *arg)
{
    struct band *b = (struct band *)arg;
    const int N = b->N;
    double *sum = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *abs_sum = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (sum == NULL || abs_sum == NULL) {
        free(sum);
        free(abs_sum);
        b->status = -2;
        return NULL;
    }
    for (int i = b->r_begin; i < b->r_end; ++i) {
        for (int j = 0; j < N; ++j) {
            sum[j] = 0.0;
            abs_sum[j] = 0.0;
        }
        /* alpha == 0: the product term is dropped and A, B are not read */
        const int nk = b->alpha != 0.0 ? b->K : 0;
        for (int k = 0; k < nk; ++k) {
            const double a = (double)b->A[(size_t)i * b->lda + k];
            const float *brow = b->B + (size_t)k * b->ldb;
            for (int j = 0; j < N; ++j) {
                const double p = a * (double)brow[j];
                sum[j] += p;
                abs_sum[j] += fabs(p);
            }
        }
        double *out = b->ref + (size_t)(i - b->row0) * N;
        double *dout = b->den + (size_t)(i - b->row0) * N;
        for (int j = 0; j < N; ++j) {
            double r = b->alpha * sum[j];
            double d = fabs(b->alpha) * abs_sum[j];
            if (b->beta != 0.0) {
                const double c = (double)b->C[(size_t)i * b->ldc + j];
                r += b->beta * c;
                d += fabs(b->beta) * fabs(c);
            }
            out[j] = r;
            dout[j] = d + ORACLE_DEN_FLOOR;
        }
    }
    free(sum);
    free(abs_sum);
    b->status = 0;
    return NULL;
}

int oracle_sgemm_rows(int M, int N, int K, float alpha, const float *A, int lda,
                      const float *B, int ldb, float beta, const float *C,
                      int ldc, int row0, int nrows, double *ref, double *den,
                      int nthreads)
{
    if (bad_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc))
        return -1;
    if (row0 < 0 || nrows < 0 || row0 > M || nrows > M - row0)
        return -1;
    if (nrows == 0 || N == 0)
        return 0;
    if (ref == NULL || den == NULL)
        return -1;
    if (nthreads <= 0)
        nthreads = oracle_nthreads();
    if (nthreads > nrows)
        nthreads = nrows;

    struct band *bands = (struct band *)calloc((size_t)nthreads, sizeof(struct band));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    int *started = (int *)calloc((size_t)nthreads, sizeof(int));
    if (bands == NULL || tids == NULL || started == NULL) {
        free(bands);
        free(tids);
        free(started);
        return -2;
    }
    int status = 0;
    for (int t = 0; t < nthreads; ++t) {
        struct band *b = &bands[t];
        b->M = M;
        b->N = N;
        b->K = K;
        b->alpha = (double)alpha;
        b->beta = (double)beta;
        b->A = A;
        b->B = B;
        b->C = C;
        b->lda = lda;
        b->ldb = ldb;
        b->ldc = ldc;
        b->row0 = row0;
        b->r_begin = row0 + (int)((long long)nrows * t / nthreads);
        b->r_end = row0 + (int)((long long)nrows * (t + 1) / nthreads);
        b->ref = ref;
        b->den = den;
        b->status = -2;
        if (pthread_create(&tids[t], NULL, run_band, b) == 0)
            started[t] = 1;
        else
            status = -2;
    }
    for (int t = 0; t < nthreads; ++t) {
        if (started[t]) {
            pthread_join(tids[t], NULL);
            if (bands[t].status != 0)
                status = bands[t].status;
        }
    }
    free(bands);
    free(tids);
    free(started);
    return status;
}

int oracle_sgemm_points(int M, int N, int K, float alpha, const float *A,
                        int lda, const float *B, int ldb, float beta,
                        const float *C, int ldc, int npts, const int *rows,
                        const int *cols, double *ref, double *den)
{
    if (bad_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc) || npts < 0)
        return -1;
    if (npts == 0)
        return 0;
    if (rows == NULL || cols == NULL || ref == NULL || den == NULL)
        return -1;
    for (int p = 0; p < npts; ++p) {
        const int i = rows[p], j = cols[p];
        if (i < 0 || i >= M || j < 0 || j >= N)
            return -1;
        double s = 0.0, s_abs = 0.0;
        /* alpha == 0: the product term is dropped and A, B are not read */
        const int kend = alpha != 0.0f ? K : 0;
        for (int k = 0; k < kend; ++k) {
            const double prod = (double)A[(size_t)i * lda + k] * (double)B[(size_t)k * ldb + j];
            s += prod;
            s_abs += fabs(prod);
        }
        double r = (double)alpha * s;
        double d = fabs((double)alpha) * s_abs;
        if (beta != 0.0f) {
            const double c = (double)C[(size_t)i * ldc + j];
            r += (double)beta * c;
            d += fabs((double)beta) * fabs(c);
        }
        ref[p] = r;
        den[p] = d + ORACLE_DEN_FLOOR;
    }
    return 0;
}
