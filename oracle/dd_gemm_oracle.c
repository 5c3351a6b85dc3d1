/*
 * ORACLE -- test infrastructure only.  Only tests/, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code with the
 * HIP path and must never be used to compute a product result for a caller.
 *
 * Classical double-double matrix product C = A·B on the CPU, the "second
 * method" of "Multiple Double Arithmetic on NVIDIA Tensor Cores", §4.2: every
 * output entry is one inner product evaluated with double-double additions and
 * multiplications.  The building blocks are the published error-free
 * transformations, written here from their definitions:
 *
 *   TwoSum (Knuth):      s = RN(a+b), e = (a+b) - s exactly, no precondition.
 *   FastTwoSum (Dekker): same result when the exponent of a is >= that of b.
 *   TwoProd (FMA):       p = RN(a*b), e = fma(a, b, -p) = a*b - p exactly.
 *   double-word + double-word: the accurate algorithm of Joldes, Muller and
 *     Popescu (ACM TOMS 44(2), 2017, "Tight and rigorous error bounds for basic
 *     building blocks of double-word arithmetic"); relative error a small
 *     multiple of u^2, u = 2^-53.
 *   double-word * double-word: the FMA-based algorithm of the same paper that
 *     keeps all three cross terms; relative error likewise O(u^2).
 *
 * Each C[i][j] accumulates its k terms in ascending k, starting from (0, 0).
 * The loop nest is i, then k, then j with a per-row accumulator, which changes
 * nothing about the order of operations on any single entry.
 *
 * Build: plain C, -ffp-contract=off (no implicit fused operations; the only
 * fused multiply-adds are the explicit fma() calls), never -ffast-math.
 * Parity status: pinned (exact rational products, identity, small integers,
 * power-of-two scaling; see tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#if defined(__FAST_MATH__)
#error "the oracle must not be built with -ffast-math"
#endif

static inline void two_sum(double a, double b, double *s, double *e) {
    double x = a + b;
    double bv = x - a;
    double av = x - bv;
    *e = (a - av) + (b - bv);
    *s = x;
}

static inline void fast_two_sum(double a, double b, double *s, double *e) {
    double x = a + b;
    *e = b - (x - a);
    *s = x;
}

static inline void two_prod(double a, double b, double *p, double *e) {
    double x = a * b;
    *e = fma(a, b, -x);
    *p = x;
}

/* (zh, zl) ~ (xh + xl) * (yh + yl) */
static inline void dd_mul(double xh, double xl, double yh, double yl,
                          double *zh, double *zl) {
    double ch, cl1;
    two_prod(xh, yh, &ch, &cl1);
    double tl0 = xl * yl;
    double tl1 = fma(xh, yl, tl0);
    double cl2 = fma(xl, yh, tl1);
    double cl3 = cl1 + cl2;
    fast_two_sum(ch, cl3, zh, zl);
}

/* (zh, zl) ~ (xh + xl) + (yh + yl) */
static inline void dd_add(double xh, double xl, double yh, double yl,
                          double *zh, double *zl) {
    double sh, sl, th, tl, vh, vl;
    two_sum(xh, yh, &sh, &sl);
    two_sum(xl, yl, &th, &tl);
    double c = sl + th;
    fast_two_sum(sh, c, &vh, &vl);
    double w = tl + vl;
    fast_two_sum(vh, w, zh, zl);
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Number of threads the OpenMP runtime will use (1 without OpenMP). */
int oracle_max_threads(void) { return set_threads(0); }

/*
 * Full product.  A is m×k (row stride lda), B is k×n (row stride ldb), C is
 * m×n (row stride ldc); all row-major float64 planes in host memory.  A lo
 * pointer may be NULL, meaning that plane is zero.  nthreads <= 0 keeps the
 * OpenMP default.  Returns the number of threads used, or -1 on bad arguments.
 */
int oracle_dd_gemm(int64_t m, int64_t n, int64_t k,
                   const double *A_hi, const double *A_lo, int64_t lda,
                   const double *B_hi, const double *B_lo, int64_t ldb,
                   double *C_hi, double *C_lo, int64_t ldc, int nthreads) {
    if (m < 0 || n < 0 || k < 0 || lda < k || ldb < n || ldc < n) return -1;
    int used = set_threads(nthreads);
#pragma omp parallel
    {
        double *acc_h = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
        double *acc_l = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < m; ++i) {
            for (int64_t j = 0; j < n; ++j) { acc_h[j] = 0.0; acc_l[j] = 0.0; }
            for (int64_t p = 0; p < k; ++p) {
                double ah = A_hi[i * lda + p];
                double al = A_lo ? A_lo[i * lda + p] : 0.0;
                const double *bh_row = B_hi + p * ldb;
                const double *bl_row = B_lo ? B_lo + p * ldb : NULL;
                for (int64_t j = 0; j < n; ++j) {
                    double ph, pl;
                    dd_mul(ah, al, bh_row[j], bl_row ? bl_row[j] : 0.0, &ph, &pl);
                    dd_add(acc_h[j], acc_l[j], ph, pl, &acc_h[j], &acc_l[j]);
                }
            }
            for (int64_t j = 0; j < n; ++j) {
                C_hi[i * ldc + j] = acc_h[j];
                C_lo[i * ldc + j] = acc_l[j];
            }
        }
        free(acc_h);
        free(acc_l);
    }
    return used;
}

/*
 * Selected entries only: out[q] = C[rows[q]][cols[q]] for q < count, each one
 * inner product in ascending k (bit-identical to the same entry of
 * oracle_dd_gemm).  Returns threads used, or -1 on bad arguments.
 */
int oracle_dd_gemm_entries(int64_t count, const int64_t *rows, const int64_t *cols,
                           int64_t m, int64_t n, int64_t k,
                           const double *A_hi, const double *A_lo, int64_t lda,
                           const double *B_hi, const double *B_lo, int64_t ldb,
                           double *out_hi, double *out_lo, int nthreads) {
    if (count < 0 || m < 0 || n < 0 || k < 0 || lda < k || ldb < n) return -1;
    for (int64_t q = 0; q < count; ++q)
        if (rows[q] < 0 || rows[q] >= m || cols[q] < 0 || cols[q] >= n) return -1;
    int used = set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t q = 0; q < count; ++q) {
        int64_t i = rows[q], j = cols[q];
        double sh = 0.0, sl = 0.0;
        for (int64_t p = 0; p < k; ++p) {
            double ph, pl;
            dd_mul(A_hi[i * lda + p], A_lo ? A_lo[i * lda + p] : 0.0,
                   B_hi[p * ldb + j], B_lo ? B_lo[p * ldb + j] : 0.0, &ph, &pl);
            dd_add(sh, sl, ph, pl, &sh, &sl);
        }
        out_hi[q] = sh;
        out_lo[q] = sl;
    }
    return used;
}

/* Scalar building blocks, exported so the tests can pin each one alone. */
void oracle_two_sum(double a, double b, double *s, double *e) { two_sum(a, b, s, e); }
void oracle_two_prod(double a, double b, double *p, double *e) { two_prod(a, b, p, e); }
void oracle_dd_mul(double xh, double xl, double yh, double yl, double *zh, double *zl) {
    dd_mul(xh, xl, yh, yl, zh, zl);
}
void oracle_dd_add(double xh, double xl, double yh, double yl, double *zh, double *zl) {
    dd_add(xh, xl, yh, yl, zh, zl);
}
