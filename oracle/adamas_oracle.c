/*
 * adamas_oracle.c -- plain, slow CPU oracle for the ADAMAS decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or table with the HIP
 * library.
 *
 * Citations refer to the ADAMAS article ("ADAMAS的核心技术解析",
 * www.lnwmold.com/news/826806) by its numbered sections:
 *   §2.1  Hadamard transform: QK^T = (HQ)(HK)^T, fast divide-and-conquer form,
 *         recursive construction of H.
 *   §2.2  dynamic three-threshold bucketing at -0.5*absmax, 0, +0.5*absmax,
 *         codes 0..3.
 *   §2.3  Manhattan distance between 2-bit codes.
 *   §3.1  compressed key cache, codes packed with left shifts 6, 4, ...
 *   §5.2  per-query token budget.
 *   §6    final attention in floating point.
 * Where the article is garbled or silent the reading used is stated at the
 * function that depends on it.
 *
 * Precision: every floating-point step is one IEEE binary32 or binary64
 * operation written out in source order; build with -O2 -ffp-contract=off
 * and without -ffast-math so that the compiler neither fuses nor reorders.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_MAX_D 4096
#define ORA_GROUP 128 /* dimensions per absmax group (§2.2 grouped quantization) */

/* Element type tags shared with the Python wrapper (not with the library). */
enum { ORA_F32 = 0, ORA_BF16 = 1 };

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one. */
static float ora_widen(const void *base, int dtype, int64_t i)
{
    if (dtype == ORA_F32)
        return ((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Correctly rounded (round-to-nearest-even) binary64 -> bf16.  Written from
 * the definition: scale the significand to 8 bits and round with rint()
 * (which rounds half-to-even in the default mode).  Going through float
 * first would double-round. */
uint16_t ora_f64_to_bf16(double x)
{
    uint64_t sbits;
    memcpy(&sbits, &x, sizeof sbits);
    uint16_t sign = (uint16_t)((sbits >> 48) & 0x8000u);
    double ax = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7fc0u);
    double r;
    if (ax < ldexp(1.0, -126)) {
        /* bf16 subnormal range: spacing 2^-133. */
        r = rint(ax * ldexp(1.0, 133)) * ldexp(1.0, -133);
    } else {
        int e;
        double m = frexp(ax, &e);              /* ax = m * 2^e, m in [0.5, 1) */
        r = ldexp(rint(m * 256.0), e - 8);     /* 8 significant bits */
    }
    float f = (float)r;                        /* exact: r has <= 8 bits */
    uint32_t fb;
    memcpy(&fb, &f, sizeof fb);
    if (isinf(f) || r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7f80u);
    return (uint16_t)(sign | (uint16_t)(fb >> 16));
}

/* ------------------------------------------------------------------------
 * §2.1 -- fast Walsh-Hadamard transform, unnormalised, Sylvester order.
 *
 * H is built by the recursion H_1 = [1], H_{2m} = [[H_m, H_m], [H_m, -H_m]]
 * (the article builds H recursively), so H[i][j] = (-1)^popcount(i&j).
 * The divide-and-conquer form applies log2(d) butterfly stages; stage h pairs
 * element i (bit h clear) with element i+h and replaces them by their sum and
 * difference.  Stages run h = 1, 2, 4, ..., d/2; each result is one binary32
 * add or subtract.  The article's orthonormal H is this transform divided by
 * sqrt(d); the codes below are invariant to that positive scale, so the
 * rounding of a 1/sqrt(d) multiply is not taken (reading: the codes come from
 * the unnormalised fp32 butterfly in this stage order).
 * ---------------------------------------------------------------------- */
void ora_fwht_f32(float *y, int d)
{
    for (int h = 1; h < d; h <<= 1) {
        for (int i = 0; i < d; i++) {
            if ((i & h) == 0) {
                float a = y[i];
                float b = y[i + h];
                y[i] = a + b;
                y[i + h] = a - b;
            }
        }
    }
}

/* Correctly rounded (round-to-nearest-even) binary64 -> binary16, returned
 * as the float of equal value (exact).  Written from the definition: 11
 * significant bits for normal results, spacing 2^-24 below 2^-14, and any
 * result above 65504 (the largest finite binary16) becomes an infinity. */
float ora_f64_to_f16_value(double x)
{
    if (isnan(x))
        return NAN;
    double ax = fabs(x), r;
    if (ax < ldexp(1.0, -14)) {
        r = rint(ax * ldexp(1.0, 24)) * ldexp(1.0, -24);
    } else {
        int e;
        double m = frexp(ax, &e);               /* ax = m * 2^e, m in [0.5, 1) */
        r = ldexp(rint(m * 2048.0), e - 11);    /* 11 significant bits */
    }
    if (r > 65504.0)
        r = INFINITY;
    return (float)copysign(r, x);
}

/* The same transform with every value in binary16 (the article's advice to
 * keep the Hadamard transform in FP16, §6): the inputs are rounded to
 * binary16, and each sum and difference is formed exactly (in binary64) and
 * rounded once to binary16. */
void ora_fwht_f16(float *y, int d)
{
    for (int i = 0; i < d; i++)
        y[i] = ora_f64_to_f16_value(y[i]);
    for (int h = 1; h < d; h <<= 1) {
        for (int i = 0; i < d; i++) {
            if ((i & h) == 0) {
                double a = y[i];
                double b = y[i + h];
                y[i] = ora_f64_to_f16_value(a + b);
                y[i + h] = ora_f64_to_f16_value(a - b);
            }
        }
    }
}

/* Same transform in binary64, divided by sqrt(d): the orthonormal H of §2.1.
 * Used only by tests of the rotation's invariants. */
void ora_hadamard_orthonormal_f64(const double *x, double *y, int d)
{
    for (int i = 0; i < d; i++)
        y[i] = x[i];
    for (int h = 1; h < d; h <<= 1)
        for (int i = 0; i < d; i++)
            if ((i & h) == 0) {
                double a = y[i], b = y[i + h];
                y[i] = a + b;
                y[i + h] = a - b;
            }
    double s = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; i++)
        y[i] *= s;
}

/* ------------------------------------------------------------------------
 * §2.2 -- three-threshold dynamic bucketing of one rotated vector.
 *
 * absmax a = max_i |y_i| over a group of dimensions (reading: the article's
 * grouped quantization, one absmax per 128 consecutive rotated dimensions of
 * one vector, i.e. per token and KV head or per query head; at head_dim <=
 * 128 the group is the whole vector).  Thresholds t0 = -0.5a, t1 = 0,
 * t2 = +0.5a, per group.  The comparison operator was lost in the article's text; the
 * reading is strict "less than":
 *     code = 0 if y < t0;  1 if y < 0;  2 if y < t2;  3 otherwise.
 * ---------------------------------------------------------------------- */
static int ora_bucket(float y, float t0, float t2)
{
    if (y < t0)
        return 0;
    if (y < 0.0f)
        return 1;
    if (y < t2)
        return 2;
    return 3;
}

/* §3.1 -- pack four 2-bit codes per byte, first code in the top bits
 * (shifts 6, 4, 2, 0 as in the article's update routine; reading: four codes
 * per byte over consecutive dimensions).  A vector of d dims -> d/4 bytes. */
static void ora_pack(const int *codes, int d, uint8_t *out)
{
    for (int j = 0; j < d / 4; j++) {
        int b = (codes[4 * j] << 6) | (codes[4 * j + 1] << 4) |
                (codes[4 * j + 2] << 2) | codes[4 * j + 3];
        out[j] = (uint8_t)b;
    }
}

/* Rotate, bucket and pack one vector given as fp32 values.  Also returns the
 * rotated values and codes when the pointers are non-null (for tests). */
/* rotate == 0 skips §2.1: the vector is bucketed as it is (the ablation row
 * "2-bit quantisation only" of the article's §3.2 table); rotate == 2 runs
 * the transform in binary16 (ora_fwht_f16).
 * alpha: the outer thresholds are -alpha*a and +alpha*a (one binary32
 * product, the lower one its negation).  §2.2 fixes alpha = 0.5; the §3.2
 * tuning list gives groups of attention heads their own bucketing thresholds,
 * read here as a per-head-group alpha (0.5 unless the caller sets one). */
void ora_encode_vec_f32_ex(const float *x, int d, int rotate, float alpha, uint8_t *packed,
                           float *y_out, int *codes_out)
{
    float y[ORA_MAX_D];
    int c[ORA_MAX_D];
    for (int i = 0; i < d; i++)
        y[i] = x[i];
    if (rotate == 2)
        ora_fwht_f16(y, d);
    else if (rotate)
        ora_fwht_f32(y, d);
    const int group = d < ORA_GROUP ? d : ORA_GROUP;
    for (int g0 = 0; g0 < d; g0 += group) {
        float a = 0.0f;
        for (int i = g0; i < g0 + group; i++) {
            float m = fabsf(y[i]);
            if (m > a)
                a = m;
        }
        float t2 = alpha * a;
        float t0 = -t2;
        for (int i = g0; i < g0 + group; i++)
            c[i] = ora_bucket(y[i], t0, t2);
    }
    ora_pack(c, d, packed);
    if (y_out)
        for (int i = 0; i < d; i++)
            y_out[i] = y[i];
    if (codes_out)
        for (int i = 0; i < d; i++)
            codes_out[i] = c[i];
}

void ora_encode_vec_f32_rot(const float *x, int d, int rotate, uint8_t *packed, float *y_out,
                            int *codes_out)
{
    ora_encode_vec_f32_ex(x, d, rotate, 0.5f, packed, y_out, codes_out);
}

void ora_encode_vec_f32(const float *x, int d, uint8_t *packed, float *y_out,
                        int *codes_out)
{
    ora_encode_vec_f32_rot(x, d, 1, packed, y_out, codes_out);
}

/* Encode keys x[batch][heads][n][d] into the code cache
 * codes[batch][heads][cap][d/4] at token rows [pos, pos+n).  Head h buckets
 * with alpha[h % n_alpha] (0.5 for every head when n_alpha == 0). */
void ora_encode_keys_ex(const void *x, int dtype, int batch, int heads, int64_t n,
                        int d, uint8_t *codes, int64_t cap, int64_t pos, int rotate,
                        const float *alpha, int n_alpha)
{
    int64_t total = (int64_t)batch * heads * n;
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < total; v++) {
        int64_t bh = v / n, t = v % n;
        int head = (int)(bh % heads);
        float a = n_alpha > 0 ? alpha[head % n_alpha] : 0.5f;
        float xv[ORA_MAX_D];
        for (int i = 0; i < d; i++)
            xv[i] = ora_widen(x, dtype, v * d + i);
        ora_encode_vec_f32_ex(xv, d, rotate, a, codes + (bh * cap + pos + t) * (d / 4), 0, 0);
    }
}

void ora_encode_keys_rot(const void *x, int dtype, int batch, int heads, int64_t n,
                         int d, uint8_t *codes, int64_t cap, int64_t pos, int rotate)
{
    ora_encode_keys_ex(x, dtype, batch, heads, n, d, codes, cap, pos, rotate, 0, 0);
}

void ora_encode_keys(const void *x, int dtype, int batch, int heads, int64_t n,
                     int d, uint8_t *codes, int64_t cap, int64_t pos)
{
    ora_encode_keys_rot(x, dtype, batch, heads, n, d, codes, cap, pos, 1);
}

/* Code i of a packed row (inverse of ora_pack). */
static int ora_code_at(const uint8_t *row, int i)
{
    return (row[i >> 2] >> (6 - 2 * (i & 3))) & 3;
}

/* §2.3 -- Manhattan distance between two packed code rows:
 * D = sum_i |qc_i - kc_i|; smaller means closer. */
uint32_t ora_manhattan(const uint8_t *qrow, const uint8_t *krow, int d)
{
    uint32_t s = 0;
    for (int i = 0; i < d; i++) {
        int diff = ora_code_at(qrow, i) - ora_code_at(krow, i);
        s += (uint32_t)(diff < 0 ? -diff : diff);
    }
    return s;
}

/* Score every cached token against every query head.  Query head hq reads KV
 * head hq / G with G = Hq / Hkv (reading: consecutive grouping).
 * q_codes[B][Hq][d/4], k_codes[B][Hkv][cap][d/4] -> dist[B][Hq][n_ctx]. */
void ora_score(const uint8_t *q_codes, const uint8_t *k_codes, int B, int Hq,
               int Hkv, int d, int64_t cap, int64_t n_ctx, uint16_t *dist)
{
    int G = Hq / Hkv;
    int rb = d / 4;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int hq = 0; hq < Hq; hq++) {
            const uint8_t *qrow = q_codes + ((int64_t)b * Hq + hq) * rb;
            const uint8_t *kbase =
                k_codes + ((int64_t)b * Hkv + hq / G) * cap * rb;
            uint16_t *drow = dist + ((int64_t)b * Hq + hq) * n_ctx;
            for (int64_t t = 0; t < n_ctx; t++)
                drow[t] = (uint16_t)ora_manhattan(qrow, kbase + t * rb, d);
        }
}

typedef struct {
    uint32_t d;
    int64_t t;
} ora_key;

static int ora_cmp_key(const void *pa, const void *pb)
{
    const ora_key *a = pa, *b = pb;
    if (a->d != b->d)
        return a->d < b->d ? -1 : 1;
    if (a->t != b->t)
        return a->t < b->t ? -1 : 1;
    return 0;
}

static int ora_cmp_i64(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* §5.2 -- token budget, with a set of tokens that is always kept.
 * The article keeps full attention for special tokens such as [CLS] (§3.2,
 * §6); the page on sparse long-context architectures pairs a sliding window
 * with attention sinks.  Reading: the first n_sink and the last n_recent of
 * the n tokens form a forced set F that ranks ahead of every other token
 * inside the budget.  For one head: order tokens by the key (0, t) for t in
 * F and (D_t + 1, t) otherwise (reading: the lowest index wins a tie), keep
 * the first min(budget, n), report them in ascending token order and pad the
 * rest of the row with -1.  With F empty this is the plain (distance, index)
 * order. */
void ora_select_row_keep(const uint16_t *drow, int64_t n, int budget, int64_t n_sink,
                         int64_t n_recent, int32_t *out)
{
    ora_key *keys = (ora_key *)malloc(sizeof(ora_key) * (size_t)(n > 0 ? n : 1));
    for (int64_t t = 0; t < n; t++) {
        int forced = t < n_sink || t >= n - n_recent;
        keys[t].d = forced ? 0u : (uint32_t)drow[t] + 1u;
        keys[t].t = t;
    }
    qsort(keys, (size_t)n, sizeof(ora_key), ora_cmp_key);
    int64_t m = n < budget ? n : budget;
    int64_t *sel = (int64_t *)malloc(sizeof(int64_t) * (size_t)(m > 0 ? m : 1));
    for (int64_t j = 0; j < m; j++)
        sel[j] = keys[j].t;
    qsort(sel, (size_t)m, sizeof(int64_t), ora_cmp_i64);
    for (int64_t j = 0; j < budget; j++)
        out[j] = j < m ? (int32_t)sel[j] : -1;
    free(sel);
    free(keys);
}

/* The plain §5.2 budget: no forced tokens. */
void ora_select_row(const uint16_t *drow, int64_t n, int budget, int32_t *out)
{
    ora_select_row_keep(drow, n, budget, 0, 0, out);
}

void ora_select_topk_keep(const uint16_t *dist, int B, int Hq, int64_t n_ctx,
                          int budget, int64_t n_sink, int64_t n_recent, int32_t *idx)
{
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; b++)
        for (int hq = 0; hq < Hq; hq++) {
            int64_t r = (int64_t)b * Hq + hq;
            ora_select_row_keep(dist + r * n_ctx, n_ctx, budget, n_sink, n_recent,
                                idx + r * (int64_t)budget);
        }
}

void ora_select_topk(const uint16_t *dist, int B, int Hq, int64_t n_ctx,
                     int budget, int32_t *idx)
{
    ora_select_topk_keep(dist, B, Hq, n_ctx, budget, 0, 0, idx);
}

/* §6 -- exact softmax attention over the selected rows only, in binary64.
 * s_j = scale * q . k_j; p = softmax(s); o = sum_j p_j v_j, using the
 * original (unrotated) q, K, V: by §2.1 the rotation leaves q.k unchanged.
 * scale == 0 means 1/sqrt(d) (reading: the usual attention scale).  Entries
 * of idx below 0 are skipped; a row with no valid entry yields zeros.  Writes
 * o in binary64 to out64 (if non-null) and rounded to the element type to
 * out.  Two error scales of a floating-point evaluation of the same
 * attention (tests bound a GPU result's error by them; neither enters o):
 * absmass64 (if non-null) receives, per output element, the sum of the
 * magnitudes of its terms, sum_j p_j |v_j,i|; scoremag64 (if non-null), per
 * (b, hq), the largest score magnitude |scale| * sum_i |q_i k_j,i| over the
 * selected rows (0 when none is selected).  Both in binary64. */
void ora_sparse_attend_ex(const void *q, const void *k, const void *v, int dtype,
                          const int32_t *idx, int B, int Hq, int Hkv, int d,
                          int64_t cap, int budget, double scale, void *out,
                          double *out64, double *absmass64, double *scoremag64)
{
    int G = Hq / Hkv;
    if (scale == 0.0)
        scale = 1.0 / sqrt((double)d);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; b++)
        for (int hq = 0; hq < Hq; hq++) {
            int64_t r = (int64_t)b * Hq + hq;
            int64_t kvbase = ((int64_t)b * Hkv + hq / G) * cap;
            const int32_t *sel = idx + r * (int64_t)budget;
            double *s = (double *)malloc(sizeof(double) * (size_t)budget);
            double o[ORA_MAX_D];
            double m = -INFINITY, smag = 0.0;
            int any = 0;
            for (int j = 0; j < budget; j++) {
                if (sel[j] < 0)
                    continue;
                int64_t row = (kvbase + sel[j]) * d;
                double acc = 0.0, mag = 0.0;
                for (int i = 0; i < d; i++) {
                    double prod = (double)ora_widen(q, dtype, r * d + i) *
                                  (double)ora_widen(k, dtype, row + i);
                    acc += prod;
                    mag += fabs(prod);
                }
                s[j] = scale * acc;
                if (s[j] > m)
                    m = s[j];
                if (fabs(scale) * mag > smag)
                    smag = fabs(scale) * mag;
                any = 1;
            }
            if (scoremag64)
                scoremag64[r] = smag;
            double am[ORA_MAX_D];
            for (int i = 0; i < d; i++) {
                o[i] = 0.0;
                am[i] = 0.0;
            }
            double l = 0.0;
            if (any) {
                for (int j = 0; j < budget; j++) {
                    if (sel[j] < 0)
                        continue;
                    double p = exp(s[j] - m);
                    l += p;
                    int64_t row = (kvbase + sel[j]) * d;
                    for (int i = 0; i < d; i++) {
                        double vi = (double)ora_widen(v, dtype, row + i);
                        o[i] += p * vi;
                        am[i] += p * fabs(vi);
                    }
                }
                for (int i = 0; i < d; i++) {
                    o[i] /= l;
                    am[i] /= l;
                }
            }
            for (int i = 0; i < d; i++) {
                if (absmass64)
                    absmass64[r * d + i] = am[i];
                if (out64)
                    out64[r * d + i] = o[i];
                if (dtype == ORA_F32)
                    ((float *)out)[r * d + i] = (float)o[i];
                else
                    ((uint16_t *)out)[r * d + i] = ora_f64_to_bf16(o[i]);
            }
            free(s);
        }
}

void ora_sparse_attend(const void *q, const void *k, const void *v, int dtype,
                       const int32_t *idx, int B, int Hq, int Hkv, int d,
                       int64_t cap, int budget, double scale, void *out,
                       double *out64)
{
    ora_sparse_attend_ex(q, k, v, dtype, idx, B, Hq, Hkv, d, cap, budget, scale, out,
                         out64, 0, 0);
}

/* One decode step for one layer: encode each query head (§2.1-§3.1), score
 * it against the first n_ctx cached codes (§2.3), keep the budget (§5.2,
 * with the forced set of ora_select_row_keep) and attend over those rows
 * (§6).  idx_out may be null. */
/* alpha / n_alpha: the per-KV-head bucketing table of ora_encode_keys_ex
 * (the keys' codes were made with it); query head hq buckets with its KV
 * head's entry, alpha[(hq / G) % n_alpha]. */
void ora_decode_step_alpha(const void *q, const void *k, const void *v,
                           const uint8_t *k_codes, int dtype, int B, int Hq, int Hkv,
                           int d, int64_t cap, int64_t n_ctx, int budget, int64_t n_sink,
                           int64_t n_recent, int rotate, const float *alpha, int n_alpha,
                           double scale, void *out, double *out64, int32_t *idx_out)
{
    int rb = d / 4;
    int G = Hq / Hkv;
    uint8_t *qc = (uint8_t *)malloc((size_t)B * Hq * rb);
    float *qalpha = (float *)malloc(sizeof(float) * (size_t)Hq);
    for (int hq = 0; hq < Hq; hq++)
        qalpha[hq] = n_alpha > 0 ? alpha[(hq / G) % n_alpha] : 0.5f;
    ora_encode_keys_ex(q, dtype, B, Hq, 1, d, qc, 1, 0, rotate, qalpha, Hq);
    free(qalpha);
    uint16_t *dist = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)B * Hq *
                                        (size_t)(n_ctx > 0 ? n_ctx : 1));
    ora_score(qc, k_codes, B, Hq, Hkv, d, cap, n_ctx, dist);
    int32_t *idx = idx_out ? idx_out
                           : (int32_t *)malloc(sizeof(int32_t) * (size_t)B * Hq *
                                               (size_t)budget);
    ora_select_topk_keep(dist, B, Hq, n_ctx, budget, n_sink, n_recent, idx);
    ora_sparse_attend(q, k, v, dtype, idx, B, Hq, Hkv, d, cap, budget, scale,
                      out, out64);
    if (!idx_out)
        free(idx);
    free(dist);
    free(qc);
}

void ora_decode_step_ex(const void *q, const void *k, const void *v,
                        const uint8_t *k_codes, int dtype, int B, int Hq, int Hkv,
                        int d, int64_t cap, int64_t n_ctx, int budget, int64_t n_sink,
                        int64_t n_recent, int rotate, double scale, void *out, double *out64,
                        int32_t *idx_out)
{
    ora_decode_step_alpha(q, k, v, k_codes, dtype, B, Hq, Hkv, d, cap, n_ctx, budget, n_sink,
                          n_recent, rotate, 0, 0, scale, out, out64, idx_out);
}

void ora_decode_step_keep(const void *q, const void *k, const void *v,
                          const uint8_t *k_codes, int dtype, int B, int Hq, int Hkv,
                          int d, int64_t cap, int64_t n_ctx, int budget, int64_t n_sink,
                          int64_t n_recent, double scale, void *out, double *out64,
                          int32_t *idx_out)
{
    ora_decode_step_ex(q, k, v, k_codes, dtype, B, Hq, Hkv, d, cap, n_ctx, budget, n_sink,
                       n_recent, 1, scale, out, out64, idx_out);
}

void ora_decode_step(const void *q, const void *k, const void *v,
                     const uint8_t *k_codes, int dtype, int B, int Hq, int Hkv,
                     int d, int64_t cap, int64_t n_ctx, int budget,
                     double scale, void *out, double *out64, int32_t *idx_out)
{
    ora_decode_step_ex(q, k, v, k_codes, dtype, B, Hq, Hkv, d, cap, n_ctx, budget, 0, 0, 1,
                       scale, out, out64, idx_out);
}
