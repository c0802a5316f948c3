/*
 * Reference GEMM oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously-correct CPU definition of the
 * operation the pgemm library computes.  It exists so that tests, the smoke
 * check and the CPU baseline leg of the benchmark can compare the GPU
 * library against something independent of it.  It shares no code, header,
 * table or helper with the HIP library, and the library never calls it.
 *
 * What it computes (the definition, written out):
 *
 *   Column-major, neither operand transposed ("optimizing-sgemm-on-nvidia-
 *   turing-gpus", introduction: column-major SGEMM with A and B not
 *   transposed).  Element (i, j) of a column-major matrix X with leading
 *   dimension ld is X[i + j*ld].  For 0 <= i < m, 0 <= j < n:
 *
 *       S(i,j) = sum_{p=0}^{k-1} A[i + p*lda] * B[p + j*ldb]
 *       R(i,j) = alpha * S(i,j) + beta * C0[i + j*ldc]
 *
 *   Row-major, as the lecture's matmat interface has it ("HPC - Lecture 13 -
 *   MatMat GPU", sections "function matmatgpu1" and "Kernel 1: Global Memory
 *   Access"): A is N1 x N2, B is N2 x N3, C is N1 x N3, row i of X starts at
 *   X + i*ld, and the kernel adds the dot product of row i of A and column j
 *   of B to C(i,j).  Written out with general alpha/beta:
 *
 *       R[i*N3 + j] = alpha * sum_p A[i*lda + p] * B[p*ldb + j]
 *                     + beta * C0[i*ldc + j]
 *
 *   The lecture's kernel has alpha = beta = 1 (it starts the sum from the
 *   old C value).  The row-major entry is written directly from this formula,
 *   not by relabelling operands, so that agreement between the two entries
 *   checks the operand-swap reading independently.
 *
 * Readings where the pages are silent (BLAS convention):
 *   - beta == 0: C0 is not read at all (NaN in C0 does not propagate).
 *   - alpha == 0 or k == 0: the product term is omitted; A and B are not read.
 *   - m == 0 or n == 0: nothing to compute.
 *
 * Arithmetic: every product and every partial sum is formed in IEEE double,
 * summed sequentially in p = 0, 1, ..., k-1 (the column-major mirror of the
 * lecture's i-k-j loop order).  For fp32 inputs each product is exact in
 * double (24 + 24 <= 53 significant bits).  Build with -ffp-contract=off so
 * that no multiply-add is fused.  The result R is returned in double and is
 * never rounded back to the input precision.
 *
 * OpenMP parallelism is over output columns (or listed entries) only; each
 * output element is computed by one thread in a fixed order, so the result
 * does not depend on the thread count.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <time.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- fp32 in */

/* R is a dense column-major m x n array of doubles with leading dimension ldr. */
void oracle_gemm_f32(int m, int n, int k, double alpha,
                     const float *A, int lda, const float *B, int ldb,
                     double beta, const float *C0, int ldc,
                     double *R, int ldr)
{
    if (m <= 0 || n <= 0) return;
    int use_ab = (k > 0 && alpha != 0.0);
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)m);
#pragma omp for schedule(static)
        for (int j = 0; j < n; ++j) {
            for (int i = 0; i < m; ++i) acc[i] = 0.0;
            if (use_ab) {
                for (int p = 0; p < k; ++p) {
                    double b = (double)B[(size_t)p + (size_t)j * ldb];
                    const float *a_col = A + (size_t)p * lda;
                    for (int i = 0; i < m; ++i)
                        acc[i] += (double)a_col[i] * b;
                }
            }
            for (int i = 0; i < m; ++i) {
                double r = use_ab ? alpha * acc[i] : 0.0;
                if (beta != 0.0) r += beta * (double)C0[(size_t)i + (size_t)j * ldc];
                R[(size_t)i + (size_t)j * ldr] = r;
            }
        }
        free(acc);
    }
}

/* R(I[t], J[t]) for t < count, one dot product per entry, same order in p. */
void oracle_gemm_f32_entries(int m, int n, int k, double alpha,
                             const float *A, int lda, const float *B, int ldb,
                             double beta, const float *C0, int ldc,
                             int count, const int64_t *I, const int64_t *J,
                             double *out)
{
    int use_ab = (k > 0 && alpha != 0.0);
    (void)m; (void)n;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < count; ++t) {
        size_t i = (size_t)I[t], j = (size_t)J[t];
        double s = 0.0;
        if (use_ab)
            for (int p = 0; p < k; ++p)
                s += (double)A[i + (size_t)p * lda] * (double)B[(size_t)p + j * ldb];
        double r = use_ab ? alpha * s : 0.0;
        if (beta != 0.0) r += beta * (double)C0[i + j * ldc];
        out[t] = r;
    }
}

/* ---------------------------------------------------------------- fp64 in */

void oracle_gemm_f64(int m, int n, int k, double alpha,
                     const double *A, int lda, const double *B, int ldb,
                     double beta, const double *C0, int ldc,
                     double *R, int ldr)
{
    if (m <= 0 || n <= 0) return;
    int use_ab = (k > 0 && alpha != 0.0);
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)m);
#pragma omp for schedule(static)
        for (int j = 0; j < n; ++j) {
            for (int i = 0; i < m; ++i) acc[i] = 0.0;
            if (use_ab) {
                for (int p = 0; p < k; ++p) {
                    double b = B[(size_t)p + (size_t)j * ldb];
                    const double *a_col = A + (size_t)p * lda;
                    for (int i = 0; i < m; ++i)
                        acc[i] += a_col[i] * b;
                }
            }
            for (int i = 0; i < m; ++i) {
                double r = use_ab ? alpha * acc[i] : 0.0;
                if (beta != 0.0) r += beta * C0[(size_t)i + (size_t)j * ldc];
                R[(size_t)i + (size_t)j * ldr] = r;
            }
        }
        free(acc);
    }
}

void oracle_gemm_f64_entries(int m, int n, int k, double alpha,
                             const double *A, int lda, const double *B, int ldb,
                             double beta, const double *C0, int ldc,
                             int count, const int64_t *I, const int64_t *J,
                             double *out)
{
    int use_ab = (k > 0 && alpha != 0.0);
    (void)m; (void)n;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < count; ++t) {
        size_t i = (size_t)I[t], j = (size_t)J[t];
        double s = 0.0;
        if (use_ab)
            for (int p = 0; p < k; ++p)
                s += A[i + (size_t)p * lda] * B[(size_t)p + j * ldb];
        double r = use_ab ? alpha * s : 0.0;
        if (beta != 0.0) r += beta * C0[i + j * ldc];
        out[t] = r;
    }
}

/* ------------------------------------------------- row-major (lecture form) */

/*
 * R is dense row-major N1 x N3 (row stride N3).  Loop order i -> p -> j with
 * a row accumulator, i.e. the lecture's i-k-j ordering, so each R(i,j) is
 * summed sequentially in p exactly like the column-major entry.
 */
void oracle_matmat_rowmajor_f64(int lda, int ldb, int ldc,
                                const double *A, const double *B,
                                const double *C0, int N1, int N2, int N3,
                                double alpha, double beta, double *R)
{
    if (N1 <= 0 || N3 <= 0) return;
    int use_ab = (N2 > 0 && alpha != 0.0);
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)N3);
#pragma omp for schedule(static)
        for (int i = 0; i < N1; ++i) {
            for (int j = 0; j < N3; ++j) acc[j] = 0.0;
            if (use_ab) {
                for (int p = 0; p < N2; ++p) {
                    double a = A[(size_t)i * lda + p];
                    const double *b_row = B + (size_t)p * ldb;
                    for (int j = 0; j < N3; ++j)
                        acc[j] += a * b_row[j];
                }
            }
            for (int j = 0; j < N3; ++j) {
                double r = use_ab ? alpha * acc[j] : 0.0;
                if (beta != 0.0) r += beta * C0[(size_t)i * ldc + j];
                R[(size_t)i * N3 + j] = r;
            }
        }
        free(acc);
    }
}

/* R(I[t], J[t]) of the row-major form for listed entries. */
void oracle_matmat_rowmajor_f64_entries(int lda, int ldb, int ldc,
                                        const double *A, const double *B,
                                        const double *C0, int N1, int N2, int N3,
                                        double alpha, double beta, int count,
                                        const int64_t *I, const int64_t *J,
                                        double *out)
{
    int use_ab = (N2 > 0 && alpha != 0.0);
    (void)N1; (void)N3;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < count; ++t) {
        size_t i = (size_t)I[t], j = (size_t)J[t];
        double s = 0.0;
        if (use_ab)
            for (int p = 0; p < N2; ++p)
                s += A[i * lda + (size_t)p] * B[(size_t)p * ldb + j];
        double r = use_ab ? alpha * s : 0.0;
        if (beta != 0.0) r += beta * C0[i * ldc + j];
        out[t] = r;
    }
}

/* ------------------------------------------------------------------ misc */

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int t)
{
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}
