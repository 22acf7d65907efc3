/*
 * ns_oracle.c -- CPU oracle for Newton-Schulz orthogonalization, fp64.
 *
 * TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
 * bench's CPU-baseline leg load this library. The GPU library does not link,
 * call or share code with it; the two have no common source, header, table or
 * helper. Plain C loops with OpenMP over output rows, no BLAS.
 *
 * What is computed. The pages name the operation but never spell it out:
 * microsoft/dion PR #74 ("Fix megabatch_orthogonalize_async hang on empty FSDP2
 * shards"), Fix section, orthogonalizes each assembled 2-D update matrix with
 * Newton-Schulz and notes that zero rows stay zero; NVIDIA/Megatron-LM PR #6379
 * ("Balance LayerWise optimizer shards by Newton-Schulz cost"), Changes item 1,
 * gives its cost as max(M,N)*min(M,N)^2. The pages give neither the
 * normalization nor the coefficients; the specification this oracle checks
 * the library against fixes the iteration, eps, the orientation, 5 steps and
 * the quintic coefficients:
 *
 *   X = G / (||G||_F + eps)                      eps = 1e-7 by default
 *   if rows > cols:  X = X^T                     (so X is m x n with m <= n)
 *   repeat `steps` times:
 *       A = X X^T                                (m x m)
 *       B = b A + c (A A)
 *       X = a X + B X
 *   if transposed:   X = X^T
 *
 * with (a, b, c) = (3.4445, -4.7750, 2.0315) supplied by the caller.
 *
 * Summation order: every sum runs over its index in increasing order, one
 * accumulator per output element, so a zero term adds exactly nothing and a
 * matrix padded with zero rows gives bitwise the same real rows.
 *
 * Parity pins for this file live in tests/test_oracle_pins.py (closed form
 * through the SVD, cubic iteration to the polar factor, zero rows/columns,
 * transposition, scaling, the singular-value band, 1x1 and 1xN cases).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define NS_ORACLE_OK 0
#define NS_ORACLE_EINVAL 1
#define NS_ORACLE_ENOMEM 3

/* ||G||_F: square root of the sum of squares, summed in row-major order. */
double ns_oracle_frobenius(const double* g, int64_t rows, int64_t cols)
{
    double s = 0.0;
    for (int64_t e = 0; e < rows * cols; ++e)
        s += g[e] * g[e];
    return sqrt(s);
}

/* dst (c x r) = src^T, src is r x c row-major. */
static void transpose(const double* src, int64_t r, int64_t c, double* dst)
{
    for (int64_t i = 0; i < r; ++i)
        for (int64_t j = 0; j < c; ++j)
            dst[j * r + i] = src[i * c + j];
}

/* A (m x m) = X X^T, X is m x n: A[i][j] = sum_k X[i][k] X[j][k]. */
static void gram(const double* x, int64_t m, int64_t n, double* a)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        const double* xi = x + i * n;
        for (int64_t j = 0; j < m; ++j) {
            const double* xj = x + j * n;
            double s = 0.0;
            for (int64_t k = 0; k < n; ++k)
                s += xi[k] * xj[k];
            a[i * m + j] = s;
        }
    }
}

/* out (m x n) = P Q, P is m x k, Q is k x n:
 * out[i][j] = sum_s P[i][s] Q[s][j], s increasing, one accumulator per element. */
static void matmul(const double* p, const double* q, int64_t m, int64_t k,
                   int64_t n, double* out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        double* oi = out + i * n;
        for (int64_t j = 0; j < n; ++j)
            oi[j] = 0.0;
        for (int64_t s = 0; s < k; ++s) {
            const double pis = p[i * k + s];
            const double* qs = q + s * n;
            for (int64_t j = 0; j < n; ++j)
                oi[j] += pis * qs[j];
        }
    }
}

/*
 * Newton-Schulz orthogonalization of one rows x cols matrix.
 *   in, out : rows*cols doubles, row-major; may alias.
 *   steps   : number of iterations (>= 0).
 *   coeffs  : coeffs[3*t + 0..2] = (a, b, c) of step t when per_step != 0,
 *             else coeffs[0..2] is used at every step.
 *   eps     : added to ||G||_F before dividing.
 * Returns 0, or 1 on invalid arguments, 3 when memory runs out.
 */
int ns_oracle_f64_sched(const double* in, double* out, int64_t rows, int64_t cols,
                        int32_t steps, const double* coeffs, int32_t per_step,
                        double eps)
{
    if (rows < 0 || cols < 0 || steps < 0 || (steps > 0 && !coeffs))
        return NS_ORACLE_EINVAL;
    if (rows == 0 || cols == 0)
        return NS_ORACLE_OK;
    if (!in || !out)
        return NS_ORACLE_EINVAL;

    const int transposed = rows > cols;
    const int64_t m = transposed ? cols : rows;
    const int64_t n = transposed ? rows : cols;

    double* x = malloc(sizeof(double) * m * n);
    double* xn = malloc(sizeof(double) * m * n);
    double* bx = malloc(sizeof(double) * m * n);
    double* a = malloc(sizeof(double) * m * m);
    double* aa = malloc(sizeof(double) * m * m);
    double* bm = malloc(sizeof(double) * m * m);
    if (!x || !xn || !bx || !a || !aa || !bm) {
        free(x); free(xn); free(bx); free(a); free(aa); free(bm);
        return NS_ORACLE_ENOMEM;
    }

    /* X = G / (||G||_F + eps), oriented so that m <= n. */
    const double scale = ns_oracle_frobenius(in, rows, cols) + eps;
    if (transposed) {
        transpose(in, rows, cols, x);
    } else {
        memcpy(x, in, sizeof(double) * m * n);
    }
    for (int64_t e = 0; e < m * n; ++e)
        x[e] = x[e] / scale;

    for (int32_t t = 0; t < steps; ++t) {
        const double* cf = per_step ? coeffs + 3 * t : coeffs;
        const double ca = cf[0], cb = cf[1], cc = cf[2];
        gram(x, m, n, a);                       /* A = X X^T        */
        matmul(a, a, m, m, m, aa);              /* A A              */
        for (int64_t e = 0; e < m * m; ++e)     /* B = b A + c A A  */
            bm[e] = cb * a[e] + cc * aa[e];
        matmul(bm, x, m, m, n, bx);             /* B X              */
        for (int64_t e = 0; e < m * n; ++e)     /* X = a X + B X    */
            xn[e] = ca * x[e] + bx[e];
        double* sw = x; x = xn; xn = sw;
    }

    if (transposed) {
        transpose(x, m, n, out);                /* back to rows x cols */
    } else {
        memcpy(out, x, sizeof(double) * m * n);
    }
    free(x); free(xn); free(bx); free(a); free(aa); free(bm);
    return NS_ORACLE_OK;
}

/* Same (a, b, c) at every step. */
int ns_oracle_f64(const double* in, double* out, int64_t rows, int64_t cols,
                  int32_t steps, const double* coeffs, double eps)
{
    return ns_oracle_f64_sched(in, out, rows, cols, steps, coeffs, 0, eps);
}
