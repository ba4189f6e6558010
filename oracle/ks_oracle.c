/*
 * ks_oracle.c -- plain fp64 CPU reference for Kronecker-sparse (KS) matrix
 * multiplication and chains of KS factors.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark load this library. The product path
 * (the HIP library and its Python binding) never links, imports or calls it,
 * and this file shares no code with it.
 *
 * What is computed.
 *   The KS abstract (taxoreview.com page "dblp:303/4794", first paragraph,
 *   opening sentence) defines a KS matrix as one whose support is a
 *   Kronecker product of identity and all-ones blocks. For the support
 *   I_a (x) 1_{b x c} (x) I_d, with the standard Kronecker index convention
 *   (the left factor varies slowest), W is (a*b*d) x (a*c*d) and its only
 *   nonzeros are
 *       W[alpha*b*d + beta*d + delta][alpha*c*d + gamma*d + delta]
 *           = K[alpha][delta][beta][gamma],
 *   for alpha < a, beta < b, gamma < c, delta < d. K is stored densely with
 *   shape (a, d, b, c), gamma fastest.
 *   The product is Y = X * W^T with X (batch x a*c*d) and Y (batch x a*b*d)
 *   both row-major, batch first, so for every row n
 *       Y[n][alpha][beta][delta] = sum_gamma K[alpha][delta][beta][gamma]
 *                                          * X[n][alpha][gamma][delta].
 *   The loop below is exactly that sum, over (n, alpha, beta, delta, gamma),
 *   in fp64, gamma ascending.
 *
 * Chains. The same abstract says KS matrices underpin Butterfly and Monarch
 * matrices, which are products of KS factors; the third paragraph of that
 * page factorises a matrix into factors with butterfly supports. A chain of
 * factors is applied in the order given: Z_0 = X, Z_{k+1} = Z_k * W_k^T, with
 * no rounding between factors (fp64 throughout).
 *
 * Inputs are fp64; callers widen fp32 or bf16 values to fp64 exactly before
 * the call. No blocking, fusion or reordering is done beyond the row-wise
 * evaluation of a chain; rows are independent and are split over OpenMP
 * threads, which does not change any result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Return codes. */
#define KS_ORACLE_OK 0
#define KS_ORACLE_BAD_ARG 1
#define KS_ORACLE_NO_MEMORY 2

static int pattern_ok(int a, int b, int c, int d) {
    return a >= 1 && b >= 1 && c >= 1 && d >= 1;
}

/* One KS factor applied to one row: y (a*b*d) from x (a*c*d). */
static void ks_factor_row(int a, int b, int c, int d, const double* K,
                          const double* x, double* y) {
    for (int alpha = 0; alpha < a; ++alpha) {
        for (int beta = 0; beta < b; ++beta) {
            for (int delta = 0; delta < d; ++delta) {
                double acc = 0.0;
                for (int gamma = 0; gamma < c; ++gamma) {
                    double k = K[(((long long)alpha * d + delta) * b + beta) * c + gamma];
                    double v = x[((long long)alpha * c + gamma) * d + delta];
                    acc += k * v;
                }
                y[((long long)alpha * b + beta) * d + delta] = acc;
            }
        }
    }
}

int ks_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Y (batch x a*b*d) = X (batch x a*c*d) * W^T for one KS factor. */
int ks_oracle_matmul(int a, int b, int c, int d, const double* K,
                     const double* X, double* Y, long long batch) {
    if (!pattern_ok(a, b, c, d) || batch < 0) return KS_ORACLE_BAD_ARG;
    if (batch == 0) return KS_ORACLE_OK;
    if (!K || !X || !Y) return KS_ORACLE_BAD_ARG;
    long long n_in = (long long)a * c * d;
    long long n_out = (long long)a * b * d;
#pragma omp parallel for schedule(static)
    for (long long n = 0; n < batch; ++n)
        ks_factor_row(a, b, c, d, K, X + n * n_in, Y + n * n_out);
    return KS_ORACLE_OK;
}

/*
 * Gradients of one factor, for the layer's backward pass. The pages give the
 * layer (a KS linear layer usable from PyTorch) but not its derivatives;
 * these are the plain chain rule on Y = X * W^T with the support above.
 * Given dY = dL/dY (batch x a*b*d):
 *   dL/dX = dY * W, i.e. for every row n
 *       dX[n][alpha][gamma][delta] = sum_beta K[alpha][delta][beta][gamma]
 *                                            * dY[n][alpha][beta][delta];
 *   dL/dK: each K[alpha][delta][beta][gamma] sits in W exactly once, at row
 *   alpha*b*d + beta*d + delta and column alpha*c*d + gamma*d + delta, so it
 *   collects that entry of dY^T * X:
 *       dK[alpha][delta][beta][gamma] = sum_n dY[n][alpha][beta][delta]
 *                                             * X[n][alpha][gamma][delta].
 * Both are evaluated exactly as written, in fp64: beta ascending for dX,
 * n ascending for dK.
 */

/* dX of one row (a*c*d) from dy (a*b*d). */
static void ks_dx_row(int a, int b, int c, int d, const double* K,
                      const double* dy, double* dx) {
    for (int alpha = 0; alpha < a; ++alpha) {
        for (int gamma = 0; gamma < c; ++gamma) {
            for (int delta = 0; delta < d; ++delta) {
                double acc = 0.0;
                for (int beta = 0; beta < b; ++beta) {
                    double k = K[(((long long)alpha * d + delta) * b + beta) * c + gamma];
                    double g = dy[((long long)alpha * b + beta) * d + delta];
                    acc += k * g;
                }
                dx[((long long)alpha * c + gamma) * d + delta] = acc;
            }
        }
    }
}

int ks_oracle_matmul_dx(int a, int b, int c, int d, const double* K,
                        const double* dY, double* dX, long long batch) {
    if (!pattern_ok(a, b, c, d) || batch < 0) return KS_ORACLE_BAD_ARG;
    if (batch == 0) return KS_ORACLE_OK;
    if (!K || !dY || !dX) return KS_ORACLE_BAD_ARG;
    long long n_in = (long long)a * c * d;
    long long n_out = (long long)a * b * d;
#pragma omp parallel for schedule(static)
    for (long long n = 0; n < batch; ++n)
        ks_dx_row(a, b, c, d, K, dY + n * n_out, dX + n * n_in);
    return KS_ORACLE_OK;
}

int ks_oracle_matmul_dw(int a, int b, int c, int d, const double* dY,
                        const double* X, double* dK, long long batch) {
    if (!pattern_ok(a, b, c, d) || batch < 0 || !dK) return KS_ORACLE_BAD_ARG;
    if (batch > 0 && (!dY || !X)) return KS_ORACLE_BAD_ARG;
    long long n_in = (long long)a * c * d;
    long long n_out = (long long)a * b * d;
    long long blocks = (long long)a * d;
#pragma omp parallel for schedule(static)
    for (long long blk = 0; blk < blocks; ++blk) {
        int alpha = (int)(blk / d), delta = (int)(blk % d);
        for (int beta = 0; beta < b; ++beta) {
            for (int gamma = 0; gamma < c; ++gamma) {
                double acc = 0.0;
                for (long long n = 0; n < batch; ++n) {
                    double g = dY[n * n_out + ((long long)alpha * b + beta) * d + delta];
                    double v = X[n * n_in + ((long long)alpha * c + gamma) * d + delta];
                    acc += g * v;
                }
                dK[(((long long)alpha * d + delta) * b + beta) * c + gamma] = acc;
            }
        }
    }
    return KS_ORACLE_OK;
}

/* Widths of a chain: width[0] = n_in of factor 0, width[k+1] = n_out of
 * factor k. Returns 0 when consecutive factors do not fit together. */
static int chain_widths(int nf, const int* pat, long long* width) {
    for (int k = 0; k < nf; ++k) {
        int a = pat[4 * k], b = pat[4 * k + 1], c = pat[4 * k + 2], d = pat[4 * k + 3];
        if (!pattern_ok(a, b, c, d)) return 0;
        long long n_in = (long long)a * c * d;
        long long n_out = (long long)a * b * d;
        if (k == 0) width[0] = n_in;
        else if (width[k] != n_in) return 0;
        width[k + 1] = n_out;
    }
    return 1;
}

/* Push one row through every factor of the chain. z0 and z1 are scratch rows
 * of at least max_width doubles; the result is written to y. */
static void chain_row(int nf, const int* pat, const double* const* Ks,
                      const long long* width, const double* x, double* y,
                      double* z0, double* z1) {
    const double* cur = x;
    for (int k = 0; k < nf; ++k) {
        double* out = (k == nf - 1) ? y : ((k % 2 == 0) ? z0 : z1);
        ks_factor_row(pat[4 * k], pat[4 * k + 1], pat[4 * k + 2], pat[4 * k + 3],
                      Ks[k], cur, out);
        cur = out;
    }
    (void)width;
}

/* Y = X * (W_{nf-1} ... W_1 W_0)^T: factor 0 is applied to X first.
 * pat holds nf patterns as (a, b, c, d) quadruples. */
int ks_oracle_chain(int nf, const int* pat, const double* const* Ks,
                    const double* X, double* Y, long long batch) {
    if (nf < 1 || !pat || !Ks || batch < 0) return KS_ORACLE_BAD_ARG;
    long long* width = (long long*)malloc(sizeof(long long) * (size_t)(nf + 1));
    if (!width) return KS_ORACLE_NO_MEMORY;
    if (!chain_widths(nf, pat, width)) { free(width); return KS_ORACLE_BAD_ARG; }
    if (batch == 0) { free(width); return KS_ORACLE_OK; }
    if (!X || !Y) { free(width); return KS_ORACLE_BAD_ARG; }
    long long maxw = 0;
    for (int k = 0; k <= nf; ++k) if (width[k] > maxw) maxw = width[k];
    int status = KS_ORACLE_OK;
#pragma omp parallel
    {
        double* z0 = (double*)malloc(sizeof(double) * (size_t)maxw);
        double* z1 = (double*)malloc(sizeof(double) * (size_t)maxw);
        if (!z0 || !z1) {
#pragma omp atomic write
            status = KS_ORACLE_NO_MEMORY;
        } else {
#pragma omp for schedule(static)
            for (long long n = 0; n < batch; ++n)
                chain_row(nf, pat, Ks, width, X + n * width[0], Y + n * width[nf], z0, z1);
        }
        free(z0);
        free(z1);
    }
    free(width);
    return status;
}

/* Compare a candidate output (float, batch x n_out of the last factor) with
 * the chain applied to X, without storing the reference output. Adds
 * sum (cand - ref)^2 to *sq_err, sum ref^2 to *sq_ref, and raises *max_abs
 * to the largest |cand - ref| seen (a NaN difference counts as infinity).
 * For a single factor pass nf = 1. */
int ks_oracle_chain_err(int nf, const int* pat, const double* const* Ks,
                        const double* X, const float* Ycand, long long batch,
                        double* sq_err, double* sq_ref, double* max_abs) {
    if (nf < 1 || !pat || !Ks || batch < 0 || !sq_err || !sq_ref || !max_abs)
        return KS_ORACLE_BAD_ARG;
    long long* width = (long long*)malloc(sizeof(long long) * (size_t)(nf + 1));
    if (!width) return KS_ORACLE_NO_MEMORY;
    if (!chain_widths(nf, pat, width)) { free(width); return KS_ORACLE_BAD_ARG; }
    if (batch == 0) { free(width); return KS_ORACLE_OK; }
    if (!X || !Ycand) { free(width); return KS_ORACLE_BAD_ARG; }
    long long maxw = 0;
    for (int k = 0; k <= nf; ++k) if (width[k] > maxw) maxw = width[k];
    long long n_out = width[nf];
    double e_sum = 0.0, r_sum = 0.0, m_abs = 0.0;
    int status = KS_ORACLE_OK;
#pragma omp parallel reduction(+ : e_sum, r_sum) reduction(max : m_abs)
    {
        double* z0 = (double*)malloc(sizeof(double) * (size_t)maxw);
        double* z1 = (double*)malloc(sizeof(double) * (size_t)maxw);
        double* y = (double*)malloc(sizeof(double) * (size_t)n_out);
        if (!z0 || !z1 || !y) {
#pragma omp atomic write
            status = KS_ORACLE_NO_MEMORY;
        } else {
#pragma omp for schedule(static)
            for (long long n = 0; n < batch; ++n) {
                chain_row(nf, pat, Ks, width, X + n * width[0], y, z0, z1);
                const float* yc = Ycand + n * n_out;
                for (long long j = 0; j < n_out; ++j) {
                    double diff = (double)yc[j] - y[j];
                    e_sum += diff * diff;
                    r_sum += y[j] * y[j];
                    double ad = fabs(diff);
                    if (isnan(ad)) ad = INFINITY;
                    if (ad > m_abs) m_abs = ad;
                }
            }
        }
        free(z0);
        free(z1);
        free(y);
    }
    free(width);
    *sq_err += e_sum;
    *sq_ref += r_sum;
    if (m_abs > *max_abs) *max_abs = m_abs;
    return status;
}
