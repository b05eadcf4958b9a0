/* Drives the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every entry point on small inputs, strided views, degenerate cases (k = 0,
 * n = 1, zero and NaN rows, duplicate generators, k = n) and argument errors.
 * Exits non-zero on a wrong status; the sanitizers abort on any memory or UB
 * error.  Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_splitmix64_stream(uint64_t seed, int64_t count, uint64_t *out);
int orc_sample_generators(int64_t n, int64_t k, uint64_t seed, int32_t *gen_idx);
int orc_gather(const void *X, int64_t n, int64_t d, int64_t ldx, int dtype, const int32_t *gen_idx, int64_t k, void *C);
int orc_compress(const void *X, int64_t n, int64_t d, int64_t ldx, int dtype, const int32_t *gen_idx, int64_t k,
                 double eps, const int64_t *rows, int64_t nrows, int32_t *f, float *alpha, double *cos_star,
                 double *margin, double *score_all);
int orc_wgrad(const void *C, int dtype, const int32_t *f, const float *alpha, int64_t n, int64_t k, int64_t d,
              const void *dY, int64_t d_out, int64_t lddy, const int64_t *cols, int64_t ncols, double *dW);
int orc_decompress(const void *C, int dtype, const int32_t *f, const float *alpha, int64_t n, int64_t k, int64_t d,
                   double *Xt64, void *Xt);
int64_t orc_footprint_bytes(int64_t n, int64_t k, int64_t d, int dtype);

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "FAILED %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static uint64_t lcg = 88172645463325252ULL;
static float frand(void) {
    lcg = lcg * 6364136223846793005ULL + 1442695040888963407ULL;
    return (float)((lcg >> 40) & 0xffffff) / 16777216.0f - 0.5f;
}

/* one full pass (sample, gather, compress, wgrad, decompress) in a dtype,
 * with X a strided view of ldx >= d columns */
static void pass(int dtype, int64_t n, int64_t d, int64_t ldx, int64_t k, int64_t dout, double eps, int special) {
    const size_t es = dtype ? 2 : 4;
    void *X = malloc((size_t)(n * ldx) * es), *dY = malloc((size_t)(n * dout) * es);
    for (int64_t i = 0; i < n * ldx; ++i) {
        float v = frand();
        if (dtype) { uint32_t b; memcpy(&b, &v, 4); ((uint16_t *)X)[i] = (uint16_t)(b >> 16); }
        else ((float *)X)[i] = v;
    }
    for (int64_t i = 0; i < n * dout; ++i) {
        float v = frand();
        if (dtype) { uint32_t b; memcpy(&b, &v, 4); ((uint16_t *)dY)[i] = (uint16_t)(b >> 16); }
        else ((float *)dY)[i] = v;
    }
    if (special && n > 4 && !dtype) {   /* zero row, NaN row, duplicate of row 0 */
        for (int64_t l = 0; l < d; ++l) {
            ((float *)X)[1 * ldx + l] = 0.0f;
            ((float *)X)[3 * ldx + l] = ((float *)X)[0 * ldx + l];
        }
        ((float *)X)[2 * ldx] = NAN;
    }
    int32_t *g = malloc(sizeof(int32_t) * (size_t)(k ? k : 1));
    EXPECT(orc_sample_generators(n, k, 1234 + (uint64_t)n, g) == 0);
    void *C = malloc((size_t)((k ? k : 1) * d) * es);
    EXPECT(orc_gather(X, n, d, ldx, dtype, g, k, C) == 0);
    int32_t *f = malloc(sizeof(int32_t) * (size_t)n);
    float *a = malloc(sizeof(float) * (size_t)n);
    double *cs = malloc(sizeof(double) * (size_t)n), *mg = malloc(sizeof(double) * (size_t)n);
    double *sc = malloc(sizeof(double) * (size_t)(n * (k ? k : 1)));
    EXPECT(orc_compress(X, n, d, ldx, dtype, g, k, eps, NULL, n, f, a, cs, mg, sc) == 0);
    int64_t rows[3] = {n - 1, 0, n / 2};
    int32_t f3[3];
    float a3[3];
    EXPECT(orc_compress(X, n, d, ldx, dtype, g, k, eps, rows, 3, f3, a3, NULL, NULL, NULL) == 0);
    EXPECT(f3[0] == f[n - 1] && f3[1] == f[0] && f3[2] == f[n / 2]);
    double *dW = malloc(sizeof(double) * (size_t)(d * dout));
    EXPECT(orc_wgrad(C, dtype, f, a, n, k, d, dY, dout, dout, NULL, dout, dW) == 0);
    int64_t cols[2] = {dout - 1, 0};
    double *dW2 = malloc(sizeof(double) * (size_t)(d * 2));
    EXPECT(orc_wgrad(C, dtype, f, a, n, k, d, dY, dout, dout, cols, 2, dW2) == 0);
    for (int64_t m = 0; m < d; ++m)   /* bitwise (a NaN generator row gives NaN entries) */
        EXPECT(!memcmp(&dW2[m * 2], &dW[m * dout + dout - 1], 8) && !memcmp(&dW2[m * 2 + 1], &dW[m * dout], 8));
    double *x64 = malloc(sizeof(double) * (size_t)(n * d));
    void *xt = malloc((size_t)(n * d) * es);
    EXPECT(orc_decompress(C, dtype, f, a, n, k, d, x64, xt) == 0);
    EXPECT(orc_footprint_bytes(n, k, d, dtype) == k * d * (int64_t)es + 8 * n);
    free(X); free(dY); free(g); free(C); free(f); free(a); free(cs); free(mg); free(sc); free(dW); free(dW2);
    free(x64); free(xt);
}

int main(void) {
    uint64_t s[5];
    EXPECT(orc_splitmix64_stream(1234567, 5, s) == 0);
    EXPECT(orc_splitmix64_stream(1, -1, s) != 0);
    int32_t g[8];
    EXPECT(orc_sample_generators(5, 6, 0, g) != 0);
    EXPECT(orc_sample_generators(5, -1, 0, g) != 0);
    EXPECT(orc_sample_generators(5, 2, 0, NULL) != 0);
    EXPECT(orc_sample_generators(0, 0, 0, NULL) == 0);
    /* argument errors */
    float x[4] = {1, 2, 3, 4};
    int32_t bad[1] = {7}, fo[2];
    float ao[2];
    EXPECT(orc_gather(x, 2, 2, 2, 0, bad, 1, x) != 0);
    EXPECT(orc_compress(x, 2, 2, 1, 0, bad, 1, 0.0, NULL, 2, fo, ao, NULL, NULL, NULL) != 0);
    EXPECT(orc_compress(x, 2, 2, 2, 0, bad, 1, 0.0, NULL, 2, fo, ao, NULL, NULL, NULL) != 0);
    EXPECT(orc_compress(x, 2, 2, 2, 0, g, 1, NAN, NULL, 2, fo, ao, NULL, NULL, NULL) != 0);
    int64_t badrow[1] = {5};
    int32_t g0[1] = {0};
    EXPECT(orc_compress(x, 2, 2, 2, 0, g0, 1, 0.0, badrow, 1, fo, ao, NULL, NULL, NULL) != 0);
    int64_t badcol[1] = {9};
    double w[4];
    EXPECT(orc_wgrad(x, 0, fo, ao, 2, 1, 2, x, 2, 2, badcol, 1, w) != 0);
    EXPECT(orc_wgrad(x, 0, fo, ao, 2, 1, 2, x, 2, 1, NULL, 2, w) != 0);
    /* passes */
    pass(0, 64, 16, 16, 8, 12, 0.3, 1);
    pass(1, 64, 16, 24, 8, 12, 0.1, 0);
    pass(0, 1, 5, 5, 1, 3, 0.5, 0);       /* n = 1 */
    pass(1, 40, 7, 8, 0, 9, 0.0, 0);      /* k = 0 */
    pass(0, 30, 6, 6, 30, 4, 0.0, 1);     /* k = n */
    pass(1, 300, 33, 40, 17, 21, 0.2, 0);
    if (fails) { fprintf(stderr, "%d failures\n", fails); return 1; }
    printf("oracle sanitizer driver ok\n");
    return 0;
}
