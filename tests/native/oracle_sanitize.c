/*
 * Drives the oracle's C functions over small seeded inputs, edge shapes
 * included (empty context, budget above the context, one row, head_dim 64 /
 * 128 / 256, both element types, sinks and recent windows, alpha tables),
 * for a build with AddressSanitizer and UndefinedBehaviorSanitizer.  It looks
 * for memory and undefined-behaviour errors only: the values are pinned by
 * the oracle's own tests.  Test infrastructure, linked with the oracle source.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t ora_f64_to_bf16(double x);
float ora_f64_to_f16_value(double x);
void ora_fwht_f32(float *y, int d);
void ora_fwht_f16(float *y, int d);
void ora_hadamard_orthonormal_f64(const double *x, double *y, int d);
void ora_encode_vec_f32_ex(const float *x, int d, int rotate, float alpha, uint8_t *packed,
                           float *y_out, int *codes_out);
void ora_encode_keys_ex(const void *x, int dtype, int batch, int heads, int64_t n, int d,
                        uint8_t *codes, int64_t cap, int64_t pos, int rotate,
                        const float *alpha, int n_alpha);
void ora_score(const uint8_t *q_codes, const uint8_t *k_codes, int B, int Hq, int Hkv, int d,
               int64_t cap, int64_t n_ctx, uint16_t *dist);
void ora_select_topk_keep(const uint16_t *dist, int B, int Hq, int64_t n_ctx, int budget,
                          int64_t n_sink, int64_t n_recent, int32_t *idx);
void ora_sparse_attend_ex(const void *q, const void *k, const void *v, int dtype,
                          const int32_t *idx, int B, int Hq, int Hkv, int d, int64_t cap,
                          int budget, double scale, void *out, double *out64, double *absmass64,
                          double *scoremag64);
void ora_decode_step_alpha(const void *q, const void *k, const void *v, const uint8_t *k_codes,
                           int dtype, int B, int Hq, int Hkv, int d, int64_t cap, int64_t n_ctx,
                           int budget, int64_t n_sink, int64_t n_recent, int rotate,
                           const float *alpha, int n_alpha, double scale, void *out,
                           double *out64, int32_t *idx_out);

static uint64_t rng_state = 0x853c49e6748fea9bull;

static double uniform01(void)
{
    /* xorshift64*: only a source of test inputs */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 2685821657736338717ull) >> 11) * 0x1.0p-53;
}

static float normal(void)
{
    double u = uniform01(), w = uniform01();
    if (u < 1e-300)
        u = 1e-300;
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * w));
}

/* n elements of the given type (0 binary32, 1 bfloat16 by truncation) */
static void *fill(int dtype, size_t n, float scale)
{
    if (dtype == 0) {
        float *p = malloc(sizeof(float) * (n ? n : 1));
        for (size_t i = 0; i < n; i++)
            p[i] = scale * normal();
        return p;
    }
    uint16_t *p = malloc(sizeof(uint16_t) * (n ? n : 1));
    for (size_t i = 0; i < n; i++) {
        float f = scale * normal();
        uint32_t b;
        memcpy(&b, &f, 4);
        p[i] = (uint16_t)(b >> 16);
    }
    return p;
}

static int run_case(int dtype, int d, int B, int Hq, int Hkv, int64_t cap, int64_t n_ctx,
                    int budget, int64_t n_sink, int64_t n_recent, int rotate, int n_alpha)
{
    const float alpha[5] = {0.25f, 0.75f, 0.5f, 0.0f, 1.5f};
    size_t es = dtype == 0 ? 4 : 2;
    void *q = fill(dtype, (size_t)B * Hq * d, 1.0f);
    void *k = fill(dtype, (size_t)B * Hkv * cap * d, 1.0f);
    void *v = fill(dtype, (size_t)B * Hkv * cap * d, 1.0f);
    uint8_t *kc = calloc((size_t)B * Hkv * cap * d / 4 + 1, 1);
    uint8_t *qc = calloc((size_t)B * Hq * d / 4 + 1, 1);
    uint16_t *dist = calloc((size_t)B * Hq * (n_ctx ? n_ctx : 1), 2);
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)B * Hq * budget);
    void *out = malloc(es * (size_t)B * Hq * d);
    double *out64 = malloc(sizeof(double) * (size_t)B * Hq * d);
    double *am = malloc(sizeof(double) * (size_t)B * Hq * d);
    double *sm = malloc(sizeof(double) * (size_t)B * Hq);

    ora_encode_keys_ex(k, dtype, B, Hkv, cap, d, kc, cap, 0, rotate, alpha, n_alpha);
    ora_encode_keys_ex(q, dtype, B, Hq, 1, d, qc, 1, 0, rotate, alpha, n_alpha);
    ora_score(qc, kc, B, Hq, Hkv, d, cap, n_ctx, dist);
    ora_select_topk_keep(dist, B, Hq, n_ctx, budget, n_sink, n_recent, idx);
    ora_sparse_attend_ex(q, k, v, dtype, idx, B, Hq, Hkv, d, cap, budget, 0.0, out, out64, am,
                         sm);
    ora_decode_step_alpha(q, k, v, kc, dtype, B, Hq, Hkv, d, cap, n_ctx, budget, n_sink,
                          n_recent, rotate, alpha, n_alpha, 0.0, out, out64, idx);
    int bad = 0;
    for (size_t i = 0; i < (size_t)B * Hq * budget; i++)
        if (idx[i] < -1 || idx[i] >= n_ctx)
            bad++;
    free(q); free(k); free(v); free(kc); free(qc); free(dist); free(idx); free(out);
    free(out64); free(am); free(sm);
    return bad;
}

int main(void)
{
    int bad = 0, cases = 0;
    const int dims[3] = {64, 128, 256};
    for (int di = 0; di < 3; di++) {
        int d = dims[di];
        float x[256], y[256];
        double xd[256], yd[256];
        uint8_t packed[64];
        int codes[256];
        for (int i = 0; i < d; i++) {
            x[i] = normal();
            xd[i] = x[i];
        }
        memcpy(y, x, sizeof(float) * d);
        ora_fwht_f32(y, d);
        memcpy(y, x, sizeof(float) * d);
        ora_fwht_f16(y, d);
        ora_hadamard_orthonormal_f64(xd, yd, d);
        for (int r = 0; r < 3; r++)
            ora_encode_vec_f32_ex(x, d, r, 0.3f, packed, y, codes);
        for (int dt = 0; dt < 2; dt++) {
            const int64_t ctxs[4] = {0, 1, 257, 300};
            for (int c = 0; c < 4; c++) {
                int64_t n = ctxs[c];
                bad += run_case(dt, d, 2, 4, 2, 300, n, 17, 0, 0, 1, 0);
                bad += run_case(dt, d, 2, 4, 2, 300, n, 300, 2, 5, 0, 3);
                bad += run_case(dt, d, 1, 3, 1, 300, n, 400, 0, 50, 2, 5);
                bad += run_case(dt, d, 2, 2, 2, 300, n, 1, 7, 0, 1, 1);
                cases += 4;
            }
        }
    }
    const double special[] = {0.0, -0.0, 1.0, -1.5, 3.4028234663852886e38, 3.4e38, 1e39, -1e39,
                              INFINITY, -INFINITY, NAN, 1e-40, -1e-45, 5e-324, 65504.0, 65520.0,
                              6e-8, 1e300};
    unsigned acc = 0;
    for (size_t i = 0; i < sizeof special / sizeof special[0]; i++) {
        acc += ora_f64_to_bf16(special[i]);
        float h = ora_f64_to_f16_value(special[i]);
        acc += isnan(h) ? 1u : 0u;
    }
    printf("oracle sanitizer run: %d cases, %d out-of-range indices (checksum %u)\n", cases, bad,
           acc);
    return bad != 0;
}
