/*
 * pamm_oracle.c -- plain, slow CPU reference for Point-Approximate Matrix
 * Multiplication (PAMM).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and this file
 * shares no code, header, table or helper with that path.
 *
 * Source of the method: the page "QKV Projections Require a Fraction of Their
 * Memory" (gist.science summary of arXiv 2506.02939), section 2
 * "Metodologia", sub-part "Algoritmo in Due Fasi":
 *   - compression (forward): k generator rows C are drawn at random from the
 *     rows of the activation matrix A; every row A_i is matched to the
 *     generator of largest cosine similarity (equivalently, smallest distance
 *     to the line that generator spans); a scale alpha_i and an index f(i)
 *     are stored so that A_i ~ alpha_i * C_f(i); a row whose approximation is
 *     too far off (tolerance epsilon) is dropped, i.e. replaced by zero; only
 *     C, f and alpha are kept;
 *   - gradient (backward): a k x m matrix B~ is formed by adding, for each
 *     generator, the output-gradient rows of its tokens weighted by alpha;
 *     the weight gradient is then approximated by C^T B~.
 * Sub-part "Scelta dei Parametri" of the same section says that removing the
 * proximity constraint altogether works best.
 *
 * Readings taken where the page leaves a step open (each is also listed in
 * the design notes of the repository):
 *   R1  similarity is the absolute cosine |<x,c>|/(|x||c|): the page allows
 *       "distance to the line spanned by C_j", and a line holds negative
 *       multiples too.
 *   R2  alpha_i = <x_i, c_f> / |c_f|^2, the least-squares scale onto that line.
 *   R3  epsilon is a similarity threshold: a row is kept iff its best
 *       |cosine| >= epsilon (so epsilon = 0 keeps every row, which is the
 *       page's "no proximity constraint"); equality keeps the row.
 *   R4  generators: k distinct rows drawn uniformly without replacement with
 *       Floyd's algorithm driven by SplitMix64, then sorted ascending.
 *   R5  ties go to the lowest generator slot; a NaN score never wins.
 *   R6  f is int32 with -1 marking a dropped row (alpha = 0 there); alpha is
 *       fp32; C keeps the input dtype.
 *   R7  a generator of zero norm scores 0; a row of zero norm has cosine 0;
 *       a row containing NaN has a NaN cosine and is dropped.
 *   R8  the argmax and the epsilon test are decided on fp32 values (each fp64
 *       score rounded once to fp32), the precision of the GPU kernel; the
 *       numbers behind the decision are computed in fp64.
 *   R9  reconstruction alpha_i * C_f(i) is formed as an fp32 product and then
 *       rounded to the storage dtype (round to nearest even).
 *
 * All arithmetic is fp64 and in plain loop order; inputs in bf16 or fp32 are
 * widened exactly.  Matrices are row-major with an explicit leading dimension
 * where the caller may pass a strided view.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_NOMEM 2

/* ------------------------------------------------------------------------ */
/* element access                                                            */
/* ------------------------------------------------------------------------ */

/* Widen one stored element to double.  A bf16 value is the top half of an
 * IEEE binary32, so the widening is exact. */
static double orc_load(const void *base, int dtype, int64_t idx) {
    if (dtype == ORC_BF16) {
        uint16_t h = ((const uint16_t *)base)[idx];
        uint32_t bits = ((uint32_t)h) << 16;
        float v;
        memcpy(&v, &bits, sizeof v);
        return (double)v;
    }
    return (double)((const float *)base)[idx];
}

static size_t orc_elem_size(int dtype) { return dtype == ORC_BF16 ? 2 : 4; }

/* Round a binary32 value to bf16, nearest-even; NaN maps to a quiet NaN. */
static uint16_t orc_f32_to_bf16(float v) {
    uint32_t bits;
    memcpy(&bits, &v, sizeof bits);
    if ((bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu) != 0)
        return (uint16_t)((bits >> 16) | 0x0040u);
    uint32_t lsb = (bits >> 16) & 1u;
    bits += 0x7fffu + lsb;
    return (uint16_t)(bits >> 16);
}

/* ------------------------------------------------------------------------ */
/* random generator selection (reading R4)                                   */
/* ------------------------------------------------------------------------ */

/* SplitMix64 (Steele, Lea and Flood 2014; public-domain reference by Vigna):
 * advance the state by the golden-ratio increment, then apply the two
 * xor-shift-multiply mixing rounds and a final xor-shift. */
static uint64_t orc_splitmix64(uint64_t *state) {
    uint64_t z = (*state += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

int orc_splitmix64_stream(uint64_t seed, int64_t count, uint64_t *out) {
    if (count < 0 || (count > 0 && !out)) return ORC_ERR_ARG;
    uint64_t s = seed;
    for (int64_t i = 0; i < count; ++i) out[i] = orc_splitmix64(&s);
    return ORC_OK;
}

/* Uniform integer in [0, m): high 64 bits of the 128-bit product. */
static uint64_t orc_below(uint64_t *state, uint64_t m) {
    unsigned __int128 p = (unsigned __int128)orc_splitmix64(state) * (unsigned __int128)m;
    return (uint64_t)(p >> 64);
}

static int orc_cmp_i32(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Floyd's sampling of k distinct values from [0, n): for j = n-k .. n-1 draw
 * t uniform in [0, j]; take t unless already taken, else take j.  The result
 * is sorted ascending, so generator slot order follows row order. */
int orc_sample_generators(int64_t n, int64_t k, uint64_t seed, int32_t *gen_idx) {
    if (n < 0 || k < 0 || k > n || n > 2147483647LL || (k > 0 && !gen_idx)) return ORC_ERR_ARG;
    if (k == 0) return ORC_OK;
    unsigned char *taken = (unsigned char *)calloc((size_t)n, 1);
    if (!taken) return ORC_ERR_NOMEM;
    uint64_t state = seed;
    int64_t cnt = 0;
    for (int64_t j = n - k; j < n; ++j) {
        int64_t t = (int64_t)orc_below(&state, (uint64_t)(j + 1));
        int64_t pick = taken[t] ? j : t;
        taken[pick] = 1;
        gen_idx[cnt++] = (int32_t)pick;
    }
    free(taken);
    qsort(gen_idx, (size_t)k, sizeof(int32_t), orc_cmp_i32);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* compression                                                               */
/* ------------------------------------------------------------------------ */

/* C_j = X[gen_idx_j]: an exact copy of the selected rows, in the input dtype. */
int orc_gather(const void *X, int64_t n, int64_t d, int64_t ldx, int dtype,
               const int32_t *gen_idx, int64_t k, void *C) {
    if (n < 0 || d < 0 || k < 0 || ldx < d) return ORC_ERR_ARG;
    size_t es = orc_elem_size(dtype);
    for (int64_t j = 0; j < k; ++j) {
        int64_t r = gen_idx[j];
        if (r < 0 || r >= n) return ORC_ERR_ARG;
        memcpy((char *)C + (size_t)(j * d) * es, (const char *)X + (size_t)(r * ldx) * es, (size_t)d * es);
    }
    return ORC_OK;
}

/*
 * Assign rows to generators (readings R1-R8).
 *
 * For each requested row i (all rows when rows == NULL, else rows[0..nrows)):
 *   dot_j   = sum_l X[i,l] * C[j,l]
 *   score_j = |dot_j| / |C_j|          (0 when |C_j| = 0)
 *   best    = lowest j maximising fp32(score_j)
 *   cos*    = score_best / |X_i|       (0 when |X_i| = 0)
 *   keep iff fp32(cos*) >= fp32(eps): f = best, alpha = fp32(dot_best/|C_best|^2)
 *   else f = -1, alpha = 0.
 * Outputs are indexed by position in the requested list.  Optional outputs
 * (NULL allowed): cos_star (fp64 best cosine), margin (fp64 gap between the
 * best and the runner-up score, in cosine units; +inf when k == 1 or the row
 * has zero norm), score_all (nrows x k fp64 cosine of every generator).
 */
int orc_compress(const void *X, int64_t n, int64_t d, int64_t ldx, int dtype,
                 const int32_t *gen_idx, int64_t k, double eps,
                 const int64_t *rows, int64_t nrows,
                 int32_t *f, float *alpha, double *cos_star, double *margin, double *score_all) {
    if (n < 0 || d < 0 || k < 0 || ldx < d || eps != eps) return ORC_ERR_ARG;
    if (!rows) nrows = n;
    if (nrows < 0) return ORC_ERR_ARG;
    if (nrows > 0 && (!f || !alpha)) return ORC_ERR_ARG;
    if (k > 0 && !gen_idx) return ORC_ERR_ARG;

    double *cn2 = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    double *dot = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    double *score = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    if (!cn2 || !dot || !score) {
        free(cn2); free(dot); free(score);
        return ORC_ERR_NOMEM;
    }
    for (int64_t j = 0; j < k; ++j) {
        int64_t r = gen_idx[j];
        if (r < 0 || r >= n) { free(cn2); free(dot); free(score); return ORC_ERR_ARG; }
        double s = 0.0;
        for (int64_t l = 0; l < d; ++l) {
            double c = orc_load(X, dtype, r * ldx + l);
            s += c * c;
        }
        cn2[j] = s;
    }
    const float eps32 = (float)eps;

    for (int64_t p = 0; p < nrows; ++p) {
        int64_t i = rows ? rows[p] : p;
        if (i < 0 || i >= n) { free(cn2); free(dot); free(score); return ORC_ERR_ARG; }
        double xn2 = 0.0;
        for (int64_t l = 0; l < d; ++l) {
            double x = orc_load(X, dtype, i * ldx + l);
            xn2 += x * x;
        }
        for (int64_t j = 0; j < k; ++j) {
            int64_t r = gen_idx[j];
            double s = 0.0;
            for (int64_t l = 0; l < d; ++l)
                s += orc_load(X, dtype, i * ldx + l) * orc_load(X, dtype, r * ldx + l);
            dot[j] = s;
            score[j] = cn2[j] > 0.0 ? fabs(s) / sqrt(cn2[j]) : 0.0;
        }
        /* argmax on fp32-rounded scores, lowest index on ties, NaN never wins */
        int64_t best = -1;
        float best32 = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            float s32 = (float)score[j];
            if (s32 != s32) continue;
            if (best < 0 || s32 > best32) { best = j; best32 = s32; }
        }
        /* cosine of the winner: 0 for a zero row (R7); a row holding NaN has
         * a NaN norm and a NaN cosine, which never passes the eps test */
        double xn = sqrt(xn2);
        double cs = 0.0;
        if (best >= 0) cs = xn2 == 0.0 ? 0.0 : score[best] / xn;
        else cs = NAN;
        int keep = (best >= 0) && ((float)cs >= eps32);
        if (keep) {
            f[p] = (int32_t)best;
            alpha[p] = cn2[best] > 0.0 ? (float)(dot[best] / cn2[best]) : 0.0f;
        } else {
            f[p] = -1;
            alpha[p] = 0.0f;
        }
        if (cos_star) cos_star[p] = cs;
        if (margin) {
            double second = -INFINITY;
            for (int64_t j = 0; j < k; ++j)
                if (j != best && score[j] == score[j] && score[j] > second) second = score[j];
            if (best < 0 || second == -INFINITY || !(xn2 > 0.0)) margin[p] = INFINITY;
            else margin[p] = (score[best] - second) / xn;
        }
        if (score_all) {
            for (int64_t j = 0; j < k; ++j)
                score_all[p * k + j] = xn2 > 0.0 ? score[j] / xn : 0.0;
        }
    }
    free(cn2); free(dot); free(score);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* approximate weight gradient                                               */
/* ------------------------------------------------------------------------ */

/*
 * B~[j, c] = sum over rows i with f(i) = j of alpha_i * dY[i, c]   (fp64)
 * dW[m, c] = sum_j C[j, m] * B~[j, c]                              (fp64)
 * Rows whose f lies outside [0, k) (the dropped marker -1) contribute
 * nothing.  Only the output columns listed in cols[0..ncols) are formed
 * (all d_out columns when cols == NULL); dW is d x ncols, row-major.
 */
int orc_wgrad(const void *C, int dtype, const int32_t *f, const float *alpha,
              int64_t n, int64_t k, int64_t d,
              const void *dY, int64_t d_out, int64_t lddy,
              const int64_t *cols, int64_t ncols, double *dW) {
    if (n < 0 || k < 0 || d < 0 || d_out < 0 || lddy < d_out) return ORC_ERR_ARG;
    if (!cols) ncols = d_out;
    if (ncols < 0) return ORC_ERR_ARG;
    if (d > 0 && ncols > 0 && !dW) return ORC_ERR_ARG;
    for (int64_t q = 0; q < ncols; ++q)
        if (cols && (cols[q] < 0 || cols[q] >= d_out)) return ORC_ERR_ARG;

    size_t gsz = (size_t)(k > 0 ? k : 1) * (size_t)(ncols > 0 ? ncols : 1);
    double *G = (double *)calloc(gsz, sizeof(double));
    if (!G) return ORC_ERR_NOMEM;
    for (int64_t i = 0; i < n; ++i) {
        int32_t j = f[i];
        if (j < 0 || j >= k) continue;
        double a = (double)alpha[i];
        for (int64_t q = 0; q < ncols; ++q) {
            int64_t c = cols ? cols[q] : q;
            G[j * ncols + q] += a * orc_load(dY, dtype, i * lddy + c);
        }
    }
    for (int64_t m = 0; m < d; ++m) {
        for (int64_t q = 0; q < ncols; ++q) {
            double s = 0.0;
            for (int64_t j = 0; j < k; ++j) s += orc_load(C, dtype, j * d + m) * G[j * ncols + q];
            dW[m * ncols + q] = s;
        }
    }
    free(G);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* reconstruction (reading R9)                                               */
/* ------------------------------------------------------------------------ */

/*
 * X~_i = alpha_i * C_f(i), or a zero row when f(i) is outside [0, k).
 * Xt64 (optional) receives the exact fp64 product; Xt (optional) receives
 * the product rounded to fp32 and then to the storage dtype.
 */
int orc_decompress(const void *C, int dtype, const int32_t *f, const float *alpha,
                   int64_t n, int64_t k, int64_t d, double *Xt64, void *Xt) {
    if (n < 0 || k < 0 || d < 0) return ORC_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) {
        int32_t j = f[i];
        int valid = (j >= 0 && j < k);
        for (int64_t l = 0; l < d; ++l) {
            double v = valid ? (double)alpha[i] * orc_load(C, dtype, (int64_t)j * d + l) : 0.0;
            if (Xt64) Xt64[i * d + l] = v;
            if (Xt) {
                float v32 = (float)v;
                if (dtype == ORC_BF16) ((uint16_t *)Xt)[i * d + l] = orc_f32_to_bf16(v32);
                else ((float *)Xt)[i * d + l] = v32;
            }
        }
    }
    return ORC_OK;
}

/* Bytes the compressed triple (C, f, alpha) occupies. */
int64_t orc_footprint_bytes(int64_t n, int64_t k, int64_t d, int dtype) {
    return k * d * (int64_t)orc_elem_size(dtype) + n * (int64_t)sizeof(int32_t) + n * (int64_t)sizeof(float);
}
