/*
 * Test infrastructure only: the plain CPU oracle for the dense symmetric /
 * Hermitian positive-definite solve (Cholesky factorization, forward and back
 * substitution, log-determinant).  Only the tests, the smoke check and the
 * benchmark's CPU baseline call it; the GPU library never does.
 *
 * What it computes (JAXMg paper, "Software design", the potrs routine): for a
 * symmetric (Hermitian) positive-definite A, the Cholesky factor A = L L^H
 * with L lower triangular and a positive real diagonal, the solution of
 * A X = B by L Y = B then L^H X = Y, and, from the same factor,
 * log det A = 2 * sum_i log L_ii.  The forward substitution L Y = B alone is
 * also exported (the Gaussian-process likelihood of the same paper, "Cholesky
 * solve (potrs)", uses it).
 *
 * The factorization is the textbook unblocked column-by-column (Crout /
 * left-looking) form of the definition L L^H = A:
 *     L_jj = sqrt(A_jj - sum_{k<j} |L_jk|^2)
 *     L_ij = (A_ij - sum_{k<j} L_ik conj(L_jk)) / L_jj        for i > j
 * There is no blocking and no reordering of the sums: every sum runs over k in
 * increasing order.  Rows of one column are independent and are spread over
 * OpenMP threads; right-hand-side columns likewise.
 *
 * Conventions (the pages are silent on them; LAPACK's are taken):
 *   - Only the lower triangle of A (j <= i) is read.  For complex A only the
 *     real part of the diagonal is read.
 *   - If the pivot A_jj - sum |L_jk|^2 is not > 0 (this includes NaN), the
 *     factorization stops and returns info = j + 1; otherwise info = 0.
 *   - Arithmetic is IEEE double (complex double for Hermitian A).
 *
 * Storage: every matrix here is a dense row-major n x n array (so the dot
 * products above run over contiguous memory); right-hand sides are stored
 * one column after another (column c at b + c*n).
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

int oracle_num_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- real --- */

/* Columns [j0, j1) of L, with the columns before j0 already in l (rows of l
 * beyond what is computed are zero).  oracle_potrf_d is this over [0, n);
 * taking the columns in several calls gives the same bits. */
int oracle_potrf_cols_d(int64_t n, const double *a, double *l, int64_t j0, int64_t j1)
{
    for (int64_t j = j0; j < j1; ++j) {
        const double *lj = l + j * n;
        double d = a[j * n + j];
        for (int64_t k = 0; k < j; ++k)
            d -= lj[k] * lj[k];
        if (!(d > 0.0))
            return (int)(j + 1);
        const double ljj = sqrt(d);
        l[j * n + j] = ljj;
#pragma omp parallel for schedule(static)
        for (int64_t i = j + 1; i < n; ++i) {
            const double *li = l + i * n;
            double s = a[i * n + j];
            for (int64_t k = 0; k < j; ++k)
                s -= li[k] * lj[k];
            l[i * n + j] = s / ljj;
        }
    }
    return 0;
}

int oracle_potrf_d(int64_t n, const double *a, double *l)
{
    memset(l, 0, sizeof(double) * (size_t)(n * n));
    return oracle_potrf_cols_d(n, a, l, 0, n);
}

/* Forward substitution L y = b (row by row), then back substitution
 * L^T x = y (column by column: once x_i is known, its contribution is removed
 * from the remaining equations 0..i-1).  b is overwritten by x. */
void oracle_potrs_d(int64_t n, int64_t nrhs, const double *l, double *b)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < nrhs; ++c) {
        double *y = b + c * n;
        for (int64_t i = 0; i < n; ++i) {
            const double *li = l + i * n;
            double s = y[i];
            for (int64_t k = 0; k < i; ++k)
                s -= li[k] * y[k];
            y[i] = s / li[i];
        }
        for (int64_t i = n - 1; i >= 0; --i) {
            const double *li = l + i * n;
            const double xi = y[i] / li[i];
            y[i] = xi;
            for (int64_t k = 0; k < i; ++k)
                y[k] -= li[k] * xi;
        }
    }
}

/* Forward substitution only: L y = b, row by row; b is overwritten by y. */
void oracle_fwd_d(int64_t n, int64_t nrhs, const double *l, double *b)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < nrhs; ++c) {
        double *y = b + c * n;
        for (int64_t i = 0; i < n; ++i) {
            const double *li = l + i * n;
            double s = y[i];
            for (int64_t k = 0; k < i; ++k)
                s -= li[k] * y[k];
            y[i] = s / li[i];
        }
    }
}

double oracle_logdet_d(int64_t n, const double *l)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += log(l[i * n + i]);
    return 2.0 * s;
}

/* ------------------------------------------------------------- complex --- */

/* Columns [j0, j1) of L, as oracle_potrf_cols_d. */
int oracle_potrf_cols_z(int64_t n, const double complex *a, double complex *l, int64_t j0, int64_t j1)
{
    for (int64_t j = j0; j < j1; ++j) {
        const double complex *lj = l + j * n;
        double d = creal(a[j * n + j]);
        for (int64_t k = 0; k < j; ++k)
            d -= creal(lj[k]) * creal(lj[k]) + cimag(lj[k]) * cimag(lj[k]);
        if (!(d > 0.0))
            return (int)(j + 1);
        const double ljj = sqrt(d);
        l[j * n + j] = ljj;
#pragma omp parallel for schedule(static)
        for (int64_t i = j + 1; i < n; ++i) {
            const double complex *li = l + i * n;
            double complex s = a[i * n + j];
            for (int64_t k = 0; k < j; ++k)
                s -= li[k] * conj(lj[k]);
            /* division of a complex number by the real pivot, part by part */
            l[i * n + j] = CMPLX(creal(s) / ljj, cimag(s) / ljj);
        }
    }
    return 0;
}

int oracle_potrf_z(int64_t n, const double complex *a, double complex *l)
{
    memset(l, 0, sizeof(double complex) * (size_t)(n * n));
    return oracle_potrf_cols_z(n, a, l, 0, n);
}

/* L y = b, then L^H x = y; b is overwritten by x. */
void oracle_potrs_z(int64_t n, int64_t nrhs, const double complex *l, double complex *b)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < nrhs; ++c) {
        double complex *y = b + c * n;
        for (int64_t i = 0; i < n; ++i) {
            const double complex *li = l + i * n;
            double complex s = y[i];
            for (int64_t k = 0; k < i; ++k)
                s -= li[k] * y[k];
            const double d = creal(li[i]);
            y[i] = CMPLX(creal(s) / d, cimag(s) / d);
        }
        for (int64_t i = n - 1; i >= 0; --i) {
            const double complex *li = l + i * n;
            const double d = creal(li[i]);
            const double complex xi = CMPLX(creal(y[i]) / d, cimag(y[i]) / d);
            y[i] = xi;
            for (int64_t k = 0; k < i; ++k)
                y[k] -= conj(li[k]) * xi;
        }
    }
}

/* Forward substitution only: L y = b; b is overwritten by y. */
void oracle_fwd_z(int64_t n, int64_t nrhs, const double complex *l, double complex *b)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < nrhs; ++c) {
        double complex *y = b + c * n;
        for (int64_t i = 0; i < n; ++i) {
            const double complex *li = l + i * n;
            double complex s = y[i];
            for (int64_t k = 0; k < i; ++k)
                s -= li[k] * y[k];
            const double d = creal(li[i]);
            y[i] = CMPLX(creal(s) / d, cimag(s) / d);
        }
    }
}

double oracle_logdet_z(int64_t n, const double complex *l)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += log(creal(l[i * n + i]));
    return 2.0 * s;
}

/* ------------------------------------------------------ single (float) --- */
/* The same three routines with every product and sum in IEEE single
 * precision (the working precision of a float32 solve); log det is summed in
 * double from the single-precision diagonal.  They time the CPU baseline of
 * float32 workloads in their own precision; parity is always checked against
 * the double-precision routines above. */

int oracle_potrf_s(int64_t n, const float *a, float *l)
{
    memset(l, 0, sizeof(float) * (size_t)(n * n));
    for (int64_t j = 0; j < n; ++j) {
        const float *lj = l + j * n;
        float d = a[j * n + j];
        for (int64_t k = 0; k < j; ++k)
            d -= lj[k] * lj[k];
        if (!(d > 0.0f))
            return (int)(j + 1);
        const float ljj = sqrtf(d);
        l[j * n + j] = ljj;
#pragma omp parallel for schedule(static)
        for (int64_t i = j + 1; i < n; ++i) {
            const float *li = l + i * n;
            float s = a[i * n + j];
            for (int64_t k = 0; k < j; ++k)
                s -= li[k] * lj[k];
            l[i * n + j] = s / ljj;
        }
    }
    return 0;
}

void oracle_potrs_s(int64_t n, int64_t nrhs, const float *l, float *b)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < nrhs; ++c) {
        float *y = b + c * n;
        for (int64_t i = 0; i < n; ++i) {
            const float *li = l + i * n;
            float s = y[i];
            for (int64_t k = 0; k < i; ++k)
                s -= li[k] * y[k];
            y[i] = s / li[i];
        }
        for (int64_t i = n - 1; i >= 0; --i) {
            const float *li = l + i * n;
            const float xi = y[i] / li[i];
            y[i] = xi;
            for (int64_t k = 0; k < i; ++k)
                y[k] -= li[k] * xi;
        }
    }
}

double oracle_logdet_s(int64_t n, const float *l)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += log((double)l[i * n + i]);
    return 2.0 * s;
}
