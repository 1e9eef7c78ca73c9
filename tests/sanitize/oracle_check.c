/* Host check of the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every entry point on exactly sized heap buffers (an out-of-bounds access faults
 * the run), on the format's and the layer's closed forms.  Test infrastructure:
 * built and run by tests/test_sanitize_host.py with gcc. */
#include "../../oracle/oracle.c"

#include <stdio.h>
#include <string.h>

static int fails = 0;
#define CHECK(c, msg) do { if (!(c)) { fprintf(stderr, "FAIL: %s\n", msg); ++fails; } } while (0)

static uint32_t rng = 0x2545F491u;
static uint32_t next(void) { rng ^= rng << 13; rng ^= rng >> 17; rng ^= rng << 5; return rng; }

/* N x K weight whose every block holds `fill` in all code bytes and f16 scale bits `d`. */
static uint8_t *weight(int64_t N, int64_t K, uint8_t fill, uint16_t d) {
    size_t nb = (size_t)N * (size_t)(K / 128) * 34;
    uint8_t *w = (uint8_t *)malloc(nb);
    for (size_t b = 0; b < nb / 34; ++b) {
        memset(w + 34 * b, fill, 32);
        w[34 * b + 32] = (uint8_t)(d & 255);
        w[34 * b + 33] = (uint8_t)(d >> 8);
    }
    return w;
}

static void tq2_cases(void) {
    const int64_t shapes[][3] = {{1, 1, 128}, {3, 40, 256}, {5, 7, 384}, {0, 4, 128}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
        int64_t M = shapes[s][0], N = shapes[s][1], K = shapes[s][2];
        size_t nb = (size_t)N * (size_t)(K / 128) * 34;
        float *x = (float *)malloc(sizeof(float) * (size_t)(M * K + 1));
        for (int64_t i = 0; i < M * K; ++i) x[i] = (float)((int32_t)next() % 1000) / 256.0f;
        double *y = (double *)malloc(sizeof(double) * (size_t)(M * N + 1));
        double *b = (double *)malloc(sizeof(double) * (size_t)(M * N + 1));
        float *y32 = (float *)malloc(sizeof(float) * (size_t)(M * N + 1));
        float *W = (float *)malloc(sizeof(float) * (size_t)(N * K));

        /* code 1 everywhere (byte 0x55): weight 0, so y = 0 and the bound is 0 */
        uint8_t *w = weight(N, K, 0x55, 0x3c00);
        CHECK(tq2_oracle_gemm(w, nb, N, K, x, M, y, b) == 0, "gemm status");
        for (int64_t i = 0; i < M * N; ++i) CHECK(y[i] == 0.0 && b[i] == 0.0, "0x55 blocks give 0");
        CHECK(tq2_oracle_dequant(w, nb, N, K, W) == 0, "dequant status");
        for (int64_t i = 0; i < N * K; ++i) CHECK(W[i] == 0.0f, "0x55 decodes to 0");
        free(w);

        /* code 0 everywhere (byte 0x00) with d = 0.5: y = -0.5 * sum_k x */
        w = weight(N, K, 0x00, 0x3800);
        CHECK(tq2_oracle_gemm(w, nb, N, K, x, M, y, b) == 0, "gemm status");
        CHECK(tq2_oracle_gemm_f32seq(w, nb, N, K, x, M, y32) == 0, "f32seq status");
        for (int64_t m = 0; m < M; ++m) {
            double sx = 0.0;
            for (int64_t k = 0; k < K; ++k) sx += x[m * K + k];
            for (int64_t n = 0; n < N; ++n) {
                CHECK(y[m * N + n] == -0.5 * sx, "0x00 blocks give -d * sum x");
                CHECK(fabs(y32[m * N + n] + 0.5 * sx) <= 1e-3 * (1.0 + fabs(sx)), "f32 reference close");
            }
        }
        if (M > 0) {
            int64_t mi[2] = {0, M - 1}, ni[2] = {N - 1, 0};
            double ya[2], ba[2];
            CHECK(tq2_oracle_gemm_at(w, nb, N, K, x, M, mi, ni, 2, ya, ba) == 0, "gemm_at status");
            CHECK(ya[0] == y[0 * N + N - 1] && ya[1] == y[(M - 1) * N], "gemm_at equals gemm");
        }
        free(w);
        /* argument errors */
        CHECK(tq2_oracle_gemm(NULL, nb, N, K, x, M, y, b) != 0, "null weight rejected");
        w = weight(1, 128, 0x00, 0x3c00);
        CHECK(tq2_oracle_dequant(w, 33, 1, 128, W) != 0, "byte count that is not N*(K/128)*34 rejected");
        free(w);
        free(x); free(y); free(b); free(y32); free(W);
    }
}

static void blr_cases(void) {
    const int64_t M = 3, d_in = 40, d_out = 24, r = 64, words = 2;
    uint32_t *bu = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(d_out * words));
    uint32_t *bv = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(d_in * words));
    float *h = (float *)malloc(sizeof(float) * d_out), *l = (float *)malloc(sizeof(float) * r);
    float *g = (float *)malloc(sizeof(float) * d_in), *x = (float *)malloc(sizeof(float) * M * d_in);
    double *y = (double *)malloc(sizeof(double) * M * d_out), *a = (double *)malloc(sizeof(double) * M * r);
    for (int64_t i = 0; i < d_out * words; ++i) bu[i] = 0xFFFFFFFFu;
    for (int64_t i = 0; i < d_in * words; ++i) bv[i] = 0xFFFFFFFFu;
    for (int64_t i = 0; i < d_out; ++i) h[i] = 0.5f + (float)i / 64.0f;
    for (int64_t i = 0; i < r; ++i) l[i] = 1.0f + (float)(i % 4) / 4.0f;
    for (int64_t i = 0; i < d_in; ++i) g[i] = 0.25f * (float)(1 + i % 3);
    for (int64_t i = 0; i < M * d_in; ++i) x[i] = (float)((int32_t)next() % 64) / 8.0f;
    CHECK(blr_oracle_forward(bu, bv, h, l, g, x, M, d_in, d_out, r, y, a) == 0, "blr status");
    double sl = 0.0;
    for (int64_t k = 0; k < r; ++k) sl += l[k];
    for (int64_t t = 0; t < M; ++t) {
        double sxg = 0.0;
        for (int64_t j = 0; j < d_in; ++j) sxg += (double)x[t * d_in + j] * (double)g[j];
        for (int64_t i = 0; i < d_out; ++i) CHECK(y[t * d_out + i] == (double)h[i] * sl * sxg, "all-ones bitmaps closed form");
        for (int64_t k = 0; k < r; ++k) CHECK(a[t * r + k] == sxg, "a = sum x.g");
    }
    int64_t ti[3] = {0, 1, 2}, ii[3] = {0, 11, 23};
    double bnd[3];
    CHECK(blr_oracle_bound_at(bu, bv, h, l, g, x, M, d_in, d_out, r, ti, ii, 3, bnd) == 0, "bound status");
    for (int s = 0; s < 3; ++s) CHECK(bnd[s] >= fabs(y[ti[s] * d_out + ii[s]]), "bound covers |y|");
    int64_t bad[1] = {M};
    CHECK(blr_oracle_bound_at(bu, bv, h, l, g, x, M, d_in, d_out, r, bad, ii, 1, bnd) != 0, "row out of range rejected");
    free(bu); free(bv); free(h); free(l); free(g); free(x); free(y); free(a);
}

int main(void) {
    oracle_set_threads(2);
    for (int i = 0; i < 65536; ++i) {  /* the f16 decode: finite values are exact and odd-symmetric */
        uint16_t hb = (uint16_t)i;
        double v = oracle_half_to_double(hb);
        if (((hb >> 10) & 31) != 31) CHECK(v == -oracle_half_to_double((uint16_t)(hb ^ 0x8000)), "f16 sign symmetry");
    }
    tq2_cases();
    blr_cases();
    if (fails) return 1;
    printf("oracle ok\n");
    return 0;
}
