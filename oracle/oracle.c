/*
 * Plain fp64 CPU oracle for the FlashOverlap one-GPU hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this file's library.  The device library shares
 * no code, header or constant with it.
 *
 * What it computes is the plain result that the method reaches faster
 * (FlashOverlap, arXiv 2604.24013):
 *   - the abstract: all-gather and reduce-scatter are replaced by decomposed
 *     peer-to-peer pieces with partitioned computation, and the result is
 *     exact, i.e. equal to the collective followed (or preceded) by the GEMM;
 *   - gist.science technical summary §1: TP/TPSP needs all-gather and
 *     reduce-scatter around the projection GEMMs, DP needs reduce-scatter;
 *   - gist.science technical summary §2: Flash-AG (gathered slices multiplied
 *     by the local weights) and Flash-RS (partial outputs summed into the shard
 *     that stays local).
 *
 * So: AG-GEMM is the unchunked product Y = X * W; GEMM-RS produces the row
 * chunks of P = X * W, and the local shard is the sum of the local partial and
 * the peers' partials; the reduce-add is the element-wise sum of R arrays.
 *
 * Arithmetic: every bf16 input is decoded exactly to double; products of two
 * bf16 values are exact in double; the GEMM sums over k in ascending order in
 * double; every reduce-add is computed exactly and rounded once to double
 * (Shewchuk's expansion summation, the method behind Python's math.fsum),
 * so no order of the terms can change it.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- bf16 <-> double ---------------------------------------------------- */

/* A bf16 value is the upper half of an IEEE binary32; decoding places the 16
 * bits in the top of a binary32 and widens it (exact). */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> bf16 bits, one rounding, to nearest with ties to even.
 * Works on the exact double value (no intermediate binary32 rounding).
 * Finite inputs whose magnitude fits bf16; overflow gives infinity. */
uint16_t oracle_f64_to_bf16(double v)
{
    if (v != v) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);               /* a = fr * 2^e with fr in [0.5, 1) */
    /* normal bf16: 8 significant bits; exponent of leading bit is e-1 */
    int lead = e - 1;
    int q;                             /* quantum exponent: ulp = 2^q */
    if (lead >= -126) q = lead - 7; else q = -133;   /* subnormal quantum */
    double scaled = ldexp(a, -q);       /* exact: a / 2^q */
    double fl = floor(scaled);
    double rem = scaled - fl;           /* exact */
    double r;
    if (rem > 0.5) r = fl + 1.0;
    else if (rem < 0.5) r = fl;
    else r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double out = ldexp(r, q);
    if (out > 3.3895313892515355e38) return sign | 0x7F80;   /* overflow */
    float f = (float)out;               /* exact: out has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

void oracle_f64_to_bf16_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(v[i]);
}

/* ---- exactly rounded summation ------------------------------------------ */

/* Returns the sum of v[0..n) rounded once to double (ties to even).
 * Shewchuk (1997): keep a list of non-overlapping partials whose exact sum is
 * the exact running sum; each new term is folded in with error-free two-sums.
 * The final step adds the partials from the largest down and fixes the one
 * case where the discarded tail sits exactly on a rounding boundary. */
double oracle_sum_exact(const double *v, int n)
{
    double stack_p[64];
    double *p = stack_p;
    int cap = 64, np = 0;
    for (int t = 0; t < n; ++t) {
        double x = v[t];
        int j = 0;
        for (int i = 0; i < np; ++i) {
            double y = p[i];
            if (fabs(x) < fabs(y)) { double tmp = x; x = y; y = tmp; }
            double hi = x + y;
            double lo = y - (hi - x);      /* exact error since |x| >= |y| */
            if (lo != 0.0) p[j++] = lo;
            x = hi;
        }
        np = j;
        if (np == cap) {
            double *q = malloc(sizeof(double) * (size_t)cap * 2);
            memcpy(q, p, sizeof(double) * (size_t)np);
            if (p != stack_p) free(p);
            p = q;
            cap *= 2;
        }
        p[np++] = x;
    }
    double hi = 0.0;
    if (np > 0) {
        int i = np - 1;
        hi = p[i];
        double lo = 0.0;
        while (i > 0) {
            double x = hi;
            double y = p[--i];
            hi = x + y;
            double yr = hi - x;
            lo = y - yr;
            if (lo != 0.0) break;
        }
        /* half-way case: the remaining partials push the tail past the tie */
        if (i > 0 && ((lo < 0.0 && p[i - 1] < 0.0) || (lo > 0.0 && p[i - 1] > 0.0))) {
            double y = lo * 2.0;
            double x = hi + y;
            double yr = x - hi;
            if (y == yr) hi = x;
        }
    }
    if (p != stack_p) free(p);
    return hi;
}

/* ---- products ----------------------------------------------------------- */

/* AG-GEMM definition: y[i][j] = sum_{t<k} x[i][t] * w[j][t], t ascending.
 * x: bf16 [m][k] row-major; w: bf16 [n][k] row-major (the K x N operand
 * stored with K contiguous); y: double [m][n]. */
void oracle_gemm(const uint16_t *x, const uint16_t *w,
                 int64_t m, int64_t n, int64_t k, double *y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < k; ++t)
                acc += oracle_bf16_to_f64(x[i * k + t]) * oracle_bf16_to_f64(w[j * k + t]);
            y[i * n + j] = acc;
        }
    }
}

/* Chunked AG-GEMM on one rank: the m rows form R chunks of m/R rows; chunks are
 * taken in the given order (any permutation of 0..R-1) and each chunk's rows
 * are multiplied by W as above.  By definition the result equals oracle_gemm. */
int oracle_ag_gemm(const uint16_t *x, const uint16_t *w,
                   int64_t m, int64_t n, int64_t k,
                   int32_t R, const int32_t *order, double *y)
{
    if (R <= 0 || m % R) return -1;
    int64_t mc = m / R;
    for (int32_t s = 0; s < R; ++s) {
        int32_t c = order[s];
        if (c < 0 || c >= R) return -1;
        oracle_gemm(x + (int64_t)c * mc * k, w, mc, n, k, y + (int64_t)c * mc * n);
    }
    return 0;
}

/* Exactly rounded element-wise sum of R fp32 arrays of n elements. */
void oracle_reduce(const float *const *srcs, int32_t R, int64_t n, double *dst)
{
    #pragma omp parallel
    {
        double *terms = malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
        #pragma omp for schedule(static)
        for (int64_t e = 0; e < n; ++e) {
            for (int32_t i = 0; i < R; ++i) terms[i] = (double)srcs[i][e];
            dst[e] = oracle_sum_exact(terms, R);
        }
        free(terms);
    }
}

/* GEMM-RS local shard: shard = P_local + sum_{q != local} incoming[q], where
 * P_local = rows of chunk `local` of X * W (double), every element summed
 * exactly.  incoming[q]: fp32 [m/R][n]; incoming[local] is ignored. */
int oracle_gemm_rs_shard(const uint16_t *x, const uint16_t *w,
                         int64_t m, int64_t n, int64_t k, int32_t R, int32_t local,
                         const float *const *incoming, double *shard)
{
    if (R <= 0 || m % R || local < 0 || local >= R) return -1;
    int64_t mc = m / R;
    double *p = malloc(sizeof(double) * (size_t)(mc * n));
    if (!p) return -2;
    oracle_gemm(x + (int64_t)local * mc * k, w, mc, n, k, p);
    #pragma omp parallel
    {
        double *terms = malloc(sizeof(double) * (size_t)R);
        #pragma omp for schedule(static)
        for (int64_t e = 0; e < mc * n; ++e) {
            int t = 0;
            terms[t++] = p[e];
            for (int32_t q = 0; q < R; ++q)
                if (q != local) terms[t++] = (double)incoming[q][e];
            shard[e] = oracle_sum_exact(terms, t);
        }
        free(terms);
    }
    free(p);
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
