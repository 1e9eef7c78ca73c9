/*
 * CPU oracle for the TQ2_0_g128 ternary-weight GEMM and the binary low-rank (BLR)
 * layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or constant with the HIP kernels.
 *
 * Plain and slow on purpose: every function is the definition written out, in
 * double precision, in ascending index order, with no blocking or reordering
 * beyond an OpenMP split over independent outputs.
 *
 * Sources (cited by page title and section):
 *  - "oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs", correctness test: a weight
 *    row is a sequence of 128-element blocks; a block is 32 bytes of 2-bit codes,
 *    four per byte with the first element in the low two bits, followed by an f16
 *    scale d; codes 0,1,2 stand for -1,0,+1, so w = (code - 1) * d; the product is
 *    out[m][n] = sum_k x[m][k] * W[n][k], stored row-major [M][N].
 *  - "cortiq-engine 0.8.43 -- train_mm.rs", module header and the `expand` kernel:
 *    W^ = diag(h) S_U diag(l) S_V^T diag(g); forward a = (x.g) S_V,
 *    c = (a.l) S_U^T, y = h.c; a sign bitmap row holds bit j of word w for rank
 *    index 32w+j, a set bit meaning +1 and a clear bit -1; bits_u has one row per
 *    output feature, bits_v one row per input feature.
 *
 * Pins: every exported function is checked by tests/test_oracle_pins.py against
 * hand-derived golden values, exact rational brute force, closed forms and
 * invariants (none is "parity unpinned").
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_OK = 0, OR_EINVAL = -1, OR_ENOMEM = -2 };

#define QBLOCK 128        /* elements per block */
#define QBLOCK_BYTES 34   /* 32 code bytes + 2 scale bytes */

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the later parallel regions (the CPU-baseline timing runs the oracle on
 * one thread and on all of them); returns the count now in force. */
int oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* IEEE 754 binary16 -> double, from the format's definition:
 * sign bit 15, exponent bits 14..10 (bias 15), fraction bits 9..0;
 * exponent 0 encodes subnormals frac * 2^-24, exponent 31 infinities and NaNs. */
double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

static int tq2_shape_ok(size_t nbytes, int64_t N, int64_t K) {
    if (N < 0 || K <= 0 || K % QBLOCK) return 0;
    return nbytes == (size_t)N * (size_t)(K / QBLOCK) * QBLOCK_BYTES;
}

/* Weight value of element k of row n (f32, exactly as the decode defines it). */
static float tq2_weight(const uint8_t *aos, int64_t K, int64_t n, int64_t k) {
    const uint8_t *blk = aos + ((size_t)n * (size_t)(K / QBLOCK) + (size_t)(k / QBLOCK)) * QBLOCK_BYTES;
    int e = (int)(k % QBLOCK);
    int code = (blk[e / 4] >> (2 * (e % 4))) & 3;
    uint16_t dbits = (uint16_t)(blk[32] | (blk[33] << 8));
    float d = (float)oracle_half_to_double(dbits);
    return (float)(code - 1) * d;
}

/* W[n][k] for the whole weight, f32 row-major [N][K]. */
int tq2_oracle_dequant(const uint8_t *aos, size_t nbytes, int64_t N, int64_t K, float *W) {
    if (!aos || !W || !tq2_shape_ok(nbytes, N, K)) return OR_EINVAL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[n * K + k] = tq2_weight(aos, K, n, k);
    return OR_OK;
}

/* One output: y = sum_k x[k]*W[n][k] in double, ascending k; bound = sum_k |x[k]*W[n][k]|. */
static void tq2_dot(const uint8_t *aos, int64_t K, int64_t n, const float *xrow, double *y, double *bound) {
    double acc = 0.0, b = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = (double)xrow[k] * (double)tq2_weight(aos, K, n, k);
        acc += p;
        b += fabs(p);
    }
    *y = acc;
    if (bound) *bound = b;
}

/* Full product: y64[M][N] and (optional) bound[M][N]. */
int tq2_oracle_gemm(const uint8_t *aos, size_t nbytes, int64_t N, int64_t K,
                    const float *x, int64_t M, double *y64, double *bound) {
    if (!aos || !x || !y64 || M < 0 || !tq2_shape_ok(nbytes, N, K)) return OR_EINVAL;
    int64_t total = M * N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = i / N, n = i % N;
        tq2_dot(aos, K, n, x + m * K, &y64[i], bound ? &bound[i] : NULL);
    }
    return OR_OK;
}

/* Selected outputs (mi[i], ni[i]) of the product; same arithmetic as the full product. */
int tq2_oracle_gemm_at(const uint8_t *aos, size_t nbytes, int64_t N, int64_t K,
                       const float *x, int64_t M, const int64_t *mi, const int64_t *ni,
                       int64_t count, double *y64, double *bound) {
    if (!aos || !x || !mi || !ni || !y64 || M < 0 || count < 0 || !tq2_shape_ok(nbytes, N, K))
        return OR_EINVAL;
    for (int64_t i = 0; i < count; ++i)
        if (mi[i] < 0 || mi[i] >= M || ni[i] < 0 || ni[i] >= N) return OR_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        tq2_dot(aos, K, ni[i], x + mi[i] * K, &y64[i], bound ? &bound[i] : NULL);
    return OR_OK;
}

/* The correctness test's own CPU reference: one f32 accumulator, acc += x*w in
 * ascending k, each product and sum rounded to f32 (no fused multiply-add). */
int tq2_oracle_gemm_f32seq(const uint8_t *aos, size_t nbytes, int64_t N, int64_t K,
                           const float *x, int64_t M, float *y32) {
    if (!aos || !x || !y32 || M < 0 || !tq2_shape_ok(nbytes, N, K)) return OR_EINVAL;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            volatile float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                volatile float p = x[m * K + k] * tq2_weight(aos, K, n, k);
                acc = acc + p;
            }
            y32[m * N + n] = acc;
        }
    return OR_OK;
}

/* ------------------------------------------------------------------ BLR layer */

/* Sign of rank index k in row `row` of a bitmap with `words` u32 per row. */
static double blr_sign(const uint32_t *bits, int64_t words, int64_t row, int64_t k) {
    return ((bits[row * words + k / 32] >> (k % 32)) & 1u) ? 1.0 : -1.0;
}

static int blr_shape_ok(int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
    return M >= 0 && d_in >= 1 && d_out >= 1 && r >= 1;
}

/* a[t][k] = sum_j x[t][j]*g[j]*S_V[j][k]  (optional output [M][r]);
 * c[t][i] = sum_k a[t][k]*l[k]*S_U[i][k];  y[t][i] = h[i]*c[t][i]   (double). */
int blr_oracle_forward(const uint32_t *bits_u, const uint32_t *bits_v,
                       const float *h, const float *l, const float *g, const float *x,
                       int64_t M, int64_t d_in, int64_t d_out, int64_t r,
                       double *y, double *a_out) {
    if (!bits_u || !bits_v || !h || !l || !g || !x || !y || !blr_shape_ok(M, d_in, d_out, r))
        return OR_EINVAL;
    int64_t words = (r + 31) / 32;
    int err = OR_OK;
#pragma omp parallel
    {
        double *a = (double *)malloc(sizeof(double) * (size_t)r);
        double *sg = (double *)malloc(sizeof(double) * (size_t)r);
        if (!a || !sg) {
#pragma omp atomic write
            err = OR_ENOMEM;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < M; ++t) {
                for (int64_t k = 0; k < r; ++k) a[k] = 0.0;
                for (int64_t j = 0; j < d_in; ++j) {       /* each a[k] sums over ascending j */
                    double xg = (double)x[t * d_in + j] * (double)g[j];
                    for (int64_t k = 0; k < r; ++k) a[k] += xg * blr_sign(bits_v, words, j, k);
                }
                if (a_out)
                    for (int64_t k = 0; k < r; ++k) a_out[t * r + k] = a[k];
                for (int64_t i = 0; i < d_out; ++i) {
                    for (int64_t k = 0; k < r; ++k) sg[k] = blr_sign(bits_u, words, i, k);
                    double c = 0.0;
                    for (int64_t k = 0; k < r; ++k) c += a[k] * (double)l[k] * sg[k];
                    y[t * d_out + i] = (double)h[i] * c;
                }
            }
        }
        free(a);
        free(sg);
    }
    return err;
}

/* Dense-equivalent magnitude bound of selected outputs (ti[s], ii[s]):
 * B = sum_j |x[t][j]| * |h[i]| * |g[j]| * |sum_k S_U[i][k]*l[k]*S_V[j][k]|. */
int blr_oracle_bound_at(const uint32_t *bits_u, const uint32_t *bits_v,
                        const float *h, const float *l, const float *g, const float *x,
                        int64_t M, int64_t d_in, int64_t d_out, int64_t r,
                        const int64_t *ti, const int64_t *ii, int64_t count, double *bound) {
    if (!bits_u || !bits_v || !h || !l || !g || !x || !ti || !ii || !bound || count < 0 ||
        !blr_shape_ok(M, d_in, d_out, r))
        return OR_EINVAL;
    for (int64_t s = 0; s < count; ++s)
        if (ti[s] < 0 || ti[s] >= M || ii[s] < 0 || ii[s] >= d_out) return OR_EINVAL;
    int64_t words = (r + 31) / 32;
#pragma omp parallel for schedule(dynamic)
    for (int64_t s = 0; s < count; ++s) {
        int64_t t = ti[s], i = ii[s];
        double b = 0.0;
        for (int64_t j = 0; j < d_in; ++j) {
            double w = 0.0;
            for (int64_t k = 0; k < r; ++k)
                w += blr_sign(bits_u, words, i, k) * (double)l[k] * blr_sign(bits_v, words, j, k);
            b += fabs((double)x[t * d_in + j]) * fabs((double)h[i]) * fabs((double)g[j]) * fabs(w);
        }
        bound[s] = b;
    }
    return OR_OK;
}
