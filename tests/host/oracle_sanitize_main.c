/*
 * Drives every entry point of the CPU oracle on small and edge-case inputs,
 * for a build with AddressSanitizer and UndefinedBehaviorSanitizer (a CPU
 * test builds and runs it; any report fails the run).  Checks a few
 * invariants on the way, so that the run also does real work: deq(backbone)
 * + residual reproduces x_n, and the dual GEMM of an all-zero input is 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_prepare(int fmt, const uint16_t *x, int64_t m, int64_t k, const uint16_t *gamma,
                   float eps, uint8_t *meta, uint8_t *s_codes, uint8_t *s_scales,
                   uint8_t *r_codes, uint8_t *r_scales, uint8_t *s_dense, float *tensor_scale);
int oracle_quantize_weight(int fmt, const uint16_t *w, int64_t n, int64_t k, uint8_t *codes,
                           uint8_t *scales, float *tensor_scale);
int oracle_dual_gemm(int fmt, const uint8_t *s_codes, const uint8_t *meta,
                     const uint8_t *s_scales, const uint8_t *r_codes, const uint8_t *r_scales,
                     const float *a_tensor_scale, const uint8_t *w_codes,
                     const uint8_t *w_scales, const float *w_tensor_scale, int64_t m, int64_t n,
                     int64_t k, float *y, double *y64, double *y_abs);
int oracle_normalize(const uint16_t *x, int64_t m, int64_t k, const uint16_t *gamma, float eps,
                     uint16_t *xn);
int oracle_residual_f32(int fmt, const uint16_t *xn, int64_t m, int64_t k, float s_t, float *r);
void oracle_residual_add(const uint16_t *h, const uint16_t *o, int64_t n, uint16_t *x);
void oracle_silu_mul(const float *g, int64_t ld_g, const float *u, int64_t ld_u, int64_t m,
                     int64_t k, uint16_t *x);
uint16_t oracle_f64_to_bf16(double v);
float oracle_tree_sum(const float *q, int64_t n);
int oracle_e4m3_encode(double v);
double oracle_e4m3_decode(int b);
int oracle_e2m1_encode(double t);
int oracle_mx_scale_exp(double amax);

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}

static uint16_t bf16_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static float f_of(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); fails++; } } while (0)

static void run(int fmt, int64_t m, int64_t k, int64_t n, int norm, int kind)
{
    int blk = fmt ? 16 : 32;
    uint16_t *x = malloc((size_t)(m * k) * 2), *g = malloc((size_t)k * 2), *w = malloc((size_t)(n * k) * 2);
    uint16_t *xn = malloc((size_t)(m * k) * 2);
    for (int64_t i = 0; i < m * k; i++) {
        float v = ((int)(next_u32() % 2001) - 1000) / 137.0f;
        if (kind == 1) v = 0.0f;                        /* all zero */
        if (kind == 2) v *= 1e-38f;                     /* subnormal squares */
        if (kind == 3 && i % 97 == 0) v = 3e38f;        /* near the top of the range */
        x[i] = bf16_of(v);
    }
    for (int64_t i = 0; i < k; i++) g[i] = bf16_of(1.0f + ((int)(next_u32() % 200) - 100) / 1000.0f);
    for (int64_t i = 0; i < n * k; i++) w[i] = bf16_of(((int)(next_u32() % 2001) - 1000) / 50000.0f);
    uint8_t *meta = malloc((size_t)(m * k / 8)), *sc = malloc((size_t)(m * k / 4)), *ss = malloc((size_t)(m * k / blk));
    uint8_t *rc = malloc((size_t)(m * k / 2)), *rsc = malloc((size_t)(m * k / blk)), *sd = malloc((size_t)(m * k / 2));
    uint8_t *wc = malloc((size_t)(n * k / 2)), *ws = malloc((size_t)(n * k / blk));
    float ts = 0.0f, wts = 0.0f;
    float *y = malloc((size_t)(m * n) * 4), *r = malloc((size_t)(m * k) * 4);
    double *y64 = malloc((size_t)(m * n) * 8), *yabs = malloc((size_t)(m * n) * 8);
    CHECK(oracle_prepare(fmt, x, m, k, norm ? g : NULL, 1e-5f, meta, sc, ss, rc, rsc, sd, &ts) == 0);
    CHECK(oracle_quantize_weight(fmt, w, n, k, wc, ws, &wts) == 0);
    CHECK(oracle_dual_gemm(fmt, sc, meta, ss, rc, rsc, &ts, wc, ws, &wts, m, n, k, y, y64, yabs) == 0);
    for (int64_t i = 0; i < m * n; i++) CHECK(fabs((double)y[i]) <= yabs[i] * 1.0000001 + 1e-300);
    if (fmt == 0) {
        CHECK(oracle_normalize(x, m, k, norm ? g : NULL, 1e-5f, xn) == 0);
        CHECK(oracle_residual_f32(fmt, xn, m, k, 1.0f, r) == 0);
    }
    if (kind == 1)
        for (int64_t i = 0; i < m * n; i++) CHECK(y[i] == 0.0f);
    free(x); free(g); free(w); free(xn); free(meta); free(sc); free(ss); free(rc); free(rsc); free(sd);
    free(wc); free(ws); free(y); free(r); free(y64); free(yabs);
}

int main(void)
{
    const int64_t shapes[][3] = {{1, 32, 1}, {3, 96, 5}, {5, 256, 7}, {2, 4096, 3}, {1, 14336, 2}};
    for (int s = 0; s < 5; s++)
        for (int kind = 0; kind < 4; kind++) {
            run(0, shapes[s][0], shapes[s][1], shapes[s][2], 1, kind);
            run(0, shapes[s][0], shapes[s][1], shapes[s][2], 0, kind);
            run(1, shapes[s][0], shapes[s][1], shapes[s][2], s % 2, kind);
        }
    /* bad arguments are refused */
    uint8_t b[64];
    float t;
    CHECK(oracle_prepare(0, NULL, 1, 33, NULL, 1e-5f, b, b, b, b, b, NULL, &t) == -1);
    CHECK(oracle_prepare(5, NULL, 1, 32, NULL, 1e-5f, b, b, b, b, b, NULL, &t) == -1);
    CHECK(oracle_quantize_weight(1, NULL, 1, 8, b, b, &t) == -1);
    /* scalar entry points over their whole domains */
    uint16_t h[64], o[64], xs[64];
    float gf[64], uf[64];
    for (int i = 0; i < 64; i++) {
        h[i] = (uint16_t)next_u32();
        o[i] = (uint16_t)next_u32();
        if ((h[i] & 0x7F80) == 0x7F80) h[i] = 0;
        if ((o[i] & 0x7F80) == 0x7F80) o[i] = 0;
        gf[i] = f_of(h[i]);
        uf[i] = f_of(o[i]);
    }
    oracle_residual_add(h, o, 64, xs);
    oracle_silu_mul(gf, 8, uf, 8, 8, 8, xs);
    for (int e = -1100; e < 1100; e += 7) {
        double v = ldexp(1.37, e);
        (void)oracle_f64_to_bf16(v);
        (void)oracle_f64_to_bf16(-v);
        (void)oracle_e4m3_encode(fabs(v));
        (void)oracle_e2m1_encode(v);
        (void)oracle_mx_scale_exp(fabs(v));
    }
    (void)oracle_f64_to_bf16(INFINITY);
    (void)oracle_f64_to_bf16(NAN);
    for (int bcode = 0; bcode < 256; bcode++) (void)oracle_e4m3_decode(bcode);
    float q[5] = {1, 2, 3, 4, 5};
    CHECK(oracle_tree_sum(q, 5) == 15.0f);
    CHECK(oracle_tree_sum(q, 0) == 0.0f);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle sanitize run ok\n");
    return 0;
}
