/*
 * oracle.c -- plain, slow fp64 CPU oracle for group-affine int4 GEMV/GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker for the HIP library; it
 * shares no code, header or constant with it.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.
 *
 * Sources (web pages, cited by title and passage):
 *   [FFAI #14] thewafflehaus/FFAI pull 14, "feat(everything-bagel): clean
 *              migration of PR #9 + #10 onto updated dev";
 *   [FFAI #9]  thewafflehaus/FFAI pull 9, "Everything Bagel".
 *
 * What is computed (restated, not quoted):
 *   - packed format: eight 4-bit codes per u32 along the input dimension, so a
 *     packed row is in_dim/8 words wide ([FFAI #14], commit adding the
 *     packed-width precondition to the batched QKV wrappers).  Code k is read
 *     from word k/8 at bit offset 4*(k%8), low nibble first: the pages do not
 *     print the nibble order, this is the plainest reading;
 *   - affine dequantisation per group of `group` input columns,
 *     w[o][k] = scale[o][k/group] * q[o][k] + bias[o][k/group]  (the int4
 *     GEMV wrappers take weight + scales + biases + in_dim + group_size,
 *     [FFAI #14] commit "dequantGemvInt4Two/Three/Four");
 *   - products: y[o] = sum_k w[o][k] * x[k] (GEMV), and for the prefill GEMM
 *     Y[t][o] = sum_k w'[o][k] * X[t][k] over the T real rows ([FFAI #9],
 *     commit introducing the dequantGemmDynamicM T-padding driver: zero rows
 *     appended, then sliced off, so padded rows never reach the result),
 *     where w' is w rounded to bfloat16 when the GEMM multiplies bf16 tiles.
 *
 * Every floating input arrives already widened (exactly) to double by the
 * Python wrapper; all arithmetic is in double, accumulated in index order.
 * No blocking, no reordering, no SIMD.  Optional OpenMP over output rows
 * only changes which thread computes a row, never the arithmetic of a row.
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <stddef.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Code k of one packed row: word k/8, nibble k%8, low nibble first. */
static unsigned code_at(const uint32_t *row_words, int64_t k)
{
    uint32_t word = row_words[k / 8];
    unsigned shift = (unsigned)(4 * (k % 8));
    return (unsigned)((word >> shift) & 15u);
}

/* Unpack rows*k_in codes into q (row-major uint8). */
void orc_unpack(const uint32_t *codes, int64_t rows, int64_t k_in, uint8_t *q)
{
    for (int64_t o = 0; o < rows; ++o)
        for (int64_t k = 0; k < k_in; ++k)
            q[o * k_in + k] = (uint8_t)code_at(codes + o * (k_in / 8), k);
}

/* One dequantised weight, exactly as the format defines it. */
static double weight_at(const uint32_t *codes, const double *scales, const double *biases,
                        int64_t o, int64_t k, int64_t k_in, int64_t group)
{
    int64_t groups = k_in / group;
    double s = scales[o * groups + k / group];
    double b = biases[o * groups + k / group];
    double q = (double)code_at(codes + o * (k_in / 8), k);
    return s * q + b;
}

/* Dequantise a whole matrix to double (rows x k_in). */
void orc_dequant(const uint32_t *codes, const double *scales, const double *biases,
                 int64_t rows, int64_t k_in, int64_t group, double *w)
{
    for (int64_t o = 0; o < rows; ++o)
        for (int64_t k = 0; k < k_in; ++k)
            w[o * k_in + k] = weight_at(codes, scales, biases, o, k, k_in, group);
}

/*
 * GEMV: y[o] = sum_k w[o][k] * x[k], plus a[o] = sum_k |w[o][k] * x[k]|
 * (the magnitude the tests use to bound fp32 accumulation noise).
 */
void orc_gemv(const uint32_t *codes, const double *scales, const double *biases,
              int64_t n_out, int64_t k_in, int64_t group, const double *x,
              double *y, double *a, int threads)
{
#ifdef _OPENMP
    if (threads < 1) threads = 1;
#pragma omp parallel for num_threads(threads) schedule(static)
#endif
    for (int64_t o = 0; o < n_out; ++o) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < k_in; ++k) {
            double term = weight_at(codes, scales, biases, o, k, k_in, group) * x[k];
            acc += term;
            mag += fabs(term);
        }
        y[o] = acc;
        if (a) a[o] = mag;
    }
    (void)threads;
}

/*
 * Magnitude product m[o] = sum_k |w[o][k]| * v[k] (v >= 0): how far an error
 * bound v on the input of a GEMV can move its output.
 */
void orc_gemv_absw(const uint32_t *codes, const double *scales, const double *biases,
                   int64_t n_out, int64_t k_in, int64_t group, const double *v,
                   double *m, int threads)
{
#ifdef _OPENMP
    if (threads < 1) threads = 1;
#pragma omp parallel for num_threads(threads) schedule(static)
#endif
    for (int64_t o = 0; o < n_out; ++o) {
        double acc = 0.0;
        for (int64_t k = 0; k < k_in; ++k)
            acc += fabs(weight_at(codes, scales, biases, o, k, k_in, group)) * v[k];
        m[o] = acc;
    }
    (void)threads;
}

/*
 * Round a double to the nearest bfloat16 value, ties to even.
 * bfloat16 keeps 8 significant bits; frexp gives v = m * 2^e with
 * 0.5 <= |m| < 1, so m * 2^8 is rounded to an integer (nearbyint honours the
 * default round-half-even mode) and scaled back.  Values here are far from
 * the bfloat16 overflow and subnormal ranges.
 */
double orc_round_bf16(double v)
{
    if (v == 0.0 || !isfinite(v)) return v;
    int e = 0;
    double m = frexp(v, &e);
    double r = nearbyint(ldexp(m, 8));
    return ldexp(r, e - 8);
}

/*
 * The prefill weight w' as the dequant GEMMs define it: the weight
 * dequantised and rounded to bfloat16 before the product (thewafflehaus/FFAI
 * pull 9, "Everything Bagel", the T-padded dequant GEMM: weights dequantised
 * to bf16, then multiplied on the matrix units).  w is the exact s * q + b
 * (exact in double: s, b float32 or bf16, q < 16), rounded once to the
 * nearest bfloat16, ties to even.
 */
static double prefill_weight(double w)
{
    return orc_round_bf16(w);
}

/* Elementwise round-to-bfloat16 of an array (in place allowed). */
void orc_round_bf16_array(const double *v, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_round_bf16(v[i]);
}

/*
 * Sampled prefill GEMM entries: for each pair i, y[i] = Y[t_idx[i]][o_idx[i]]
 *   = sum_k w'[o][k] * X[t][k], with w' = prefill_weight(w) when round_w != 0,
 * else the exact w.  X is T x ldx (row-major, doubles).
 */
void orc_gemm_entries(const uint32_t *codes, const double *scales, const double *biases,
                      int64_t n_out, int64_t k_in, int64_t group, const double *X, int64_t ldx,
                      const int64_t *t_idx, const int64_t *o_idx, int64_t n_pairs,
                      int round_w, double *y, double *a, int threads)
{
#ifdef _OPENMP
    if (threads < 1) threads = 1;
#pragma omp parallel for num_threads(threads) schedule(static)
#endif
    for (int64_t i = 0; i < n_pairs; ++i) {
        int64_t t = t_idx[i], o = o_idx[i];
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < k_in; ++k) {
            double w = weight_at(codes, scales, biases, o, k, k_in, group);
            if (round_w) w = prefill_weight(w);
            double term = w * X[t * ldx + k];
            acc += term;
            mag += fabs(term);
        }
        y[i] = acc;
        if (a) a[i] = mag;
    }
    (void)threads;
    (void)n_out;
}

/*
 * Full prefill GEMM over all T x n_out entries.  Each row of w' is
 * dequantised once into a buffer and then multiplied with every X row; every
 * entry is still the plain index-order sum over k.  Returns -1 if the row
 * buffer cannot be allocated, 0 otherwise.
 */
int orc_gemm(const uint32_t *codes, const double *scales, const double *biases,
             int64_t n_out, int64_t k_in, int64_t group, const double *X, int64_t T,
             int round_w, double *Y, double *A, int threads)
{
    int failed = 0;
#ifdef _OPENMP
    if (threads < 1) threads = 1;
#pragma omp parallel num_threads(threads) reduction(|:failed)
#endif
    {
        double *wrow = (double *)malloc((size_t)k_in * sizeof(double));
        if (!wrow) failed = 1;
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t o = 0; o < n_out; ++o) {
            if (!wrow) continue;
            for (int64_t k = 0; k < k_in; ++k) {
                double w = weight_at(codes, scales, biases, o, k, k_in, group);
                wrow[k] = round_w ? prefill_weight(w) : w;
            }
            for (int64_t t = 0; t < T; ++t) {
                const double *x = X + t * k_in;
                double acc = 0.0, mag = 0.0;
                for (int64_t k = 0; k < k_in; ++k) {
                    double term = wrow[k] * x[k];
                    acc += term;
                    mag += fabs(term);
                }
                Y[t * n_out + o] = acc;
                if (A) A[t * n_out + o] = mag;
            }
        }
        free(wrow);
    }
    (void)threads;
    return failed ? -1 : 0;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
