/*
 * SharQ CPU oracle.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the product path never does.
 *
 * A plain, slow statement of what the SharQ linear-layer path computes
 * (single-threaded as the tests build it; the benchmark's CPU baseline also
 * builds it with OpenMP, which runs independent rows on threads and changes
 * no value), following "SharQ: Bridging Activation Sparsity and FP4
 * Quantization for LLM Inference" (arXiv:2606.26587), abstract:
 *   sentence 3: an input-adaptive N:M mask extracts an outlier-dominated
 *               sparse backbone, which is quantized to FP4; the dense
 *               residual is taken against the QUANTIZED backbone;
 *   sentence 4: a sparse FP4 GEMM on the backbone plus a dense FP4 GEMM on
 *               the residual;
 *   sentence 5: one FP4 weight payload read by both paths; the preparation
 *               step also applies the layer normalization;
 *   sentence 7: NVFP4 and MXFP4 formats.
 * Concrete choices the abstract leaves open (2:4 along K, RMSNorm, block 32
 * with E8M0 scales for MXFP4, block 16 with E4M3 scales and an fp32 tensor
 * scale for NVFP4, the tie-break, rounding of every fp32 step) are the
 * readings listed in the design notes; each function below names the one it
 * takes.  Value rules for E2M1, E8M0 and E4M3 are those of the OCP
 * Microscaling v1.0 and OCP 8-bit floating point specifications.
 *
 * Every fp32 step is written as a C float operation (IEEE binary32, round to
 * nearest even; the file is built with -ffp-contract=off, no fast-math, and
 * denormals are kept).  Quantization decisions on values that are exact in
 * binary32 are taken on the exact value, in double.
 *
 * Shares no code with the HIP path.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MXFP4 0
#define ORACLE_NVFP4 1

/* ------------------------------------------------------------------ */
/* bfloat16 <-> float                                                  */
/* ------------------------------------------------------------------ */

float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a finite float to the nearest bfloat16, ties to even. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7FFFu + keep_lsb;
    return (uint16_t)(u >> 16);
}

/*
 * A bf16 output of the dual GEMM: each fp32 value of Y rounded to bf16 once,
 * to nearest with ties to even (oracle_f32_to_bf16).  Reading: the abstract
 * (sentence 4) sums both paths into one fp32-accumulated output; a bf16
 * output is that fp32 sum rounded once, which is what storing the fp32
 * result in bf16 gives.  Y is finite here, so no NaN or overflow case arises.
 */
void oracle_round_bf16(const float *y, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(y[i]);
}

/* ------------------------------------------------------------------ */
/* Element and scale codecs (OCP MX v1.0 E2M1 / E8M0, OCP FP8 E4M3)     */
/* ------------------------------------------------------------------ */

/* E2M1 magnitudes by 3-bit code: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_decode(int code)
{
    double v = e2m1_mag[code & 7];
    return (code & 8) ? -v : v;
}

/*
 * E2M1 code of t: round to nearest representable magnitude, ties to the
 * code whose mantissa bit is 0 (the even code), saturating at 6.  The sign
 * bit follows the sign of t, also when the magnitude rounds to zero.
 * The midpoints between neighbours are 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.
 */
int oracle_e2m1_encode(double t)
{
    int sign = signbit(t) ? 8 : 0;
    double a = fabs(t);
    int m;
    if (a <= 0.25)      m = 0;   /* tie 0.25 -> 0 (even) */
    else if (a < 0.75)  m = 1;   /* tie 0.75 -> 1.0 (even) */
    else if (a <= 1.25) m = 2;   /* tie 1.25 -> 1.0 (even) */
    else if (a < 1.75)  m = 3;   /* tie 1.75 -> 2.0 (even) */
    else if (a <= 2.5)  m = 4;   /* tie 2.5 -> 2.0 (even) */
    else if (a < 3.5)   m = 5;   /* tie 3.5 -> 4.0 (even) */
    else if (a <= 5.0)  m = 6;   /* tie 5 -> 4.0 (even) */
    else                m = 7;   /* saturate to 6 */
    return sign | m;
}

/*
 * MX shared scale exponent for a block whose largest magnitude is amax:
 * floor(log2(amax)) minus the largest E2M1 exponent (2), clamped to the
 * E8M0 range [-127, 127]; amax = 0 gives -127.  The E8M0 byte is e + 127.
 */
int oracle_mx_scale_exp(double amax)
{
    if (amax == 0.0)
        return -127;
    int E;
    frexp(amax, &E);       /* amax = f * 2^E with f in [0.5, 1) */
    E -= 1;                /* now amax = f' * 2^E with f' in [1, 2) */
    int e = E - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/*
 * OCP FP8 E4M3 code of a non-negative finite value: bias 7, 3 mantissa bits,
 * subnormals down to 2^-9, round to nearest even, saturating to the largest
 * finite value 448 (code 0x7E).  0x7F (NaN) is never produced.
 */
int oracle_e4m3_encode(double v)
{
    if (!(v > 0.0))
        return 0;
    if (v >= 448.0)
        return 0x7E;
    int E;
    frexp(v, &E);
    E -= 1;                                /* v = f * 2^E, f in [1, 2) */
    if (E < -6) {                          /* subnormal: multiples of 2^-9 */
        double q = nearbyint(v * 512.0);   /* 0..8; 8 is the smallest normal */
        return (int)q;
    }
    double f = ldexp(v, -E);               /* [1, 2) */
    int m = (int)nearbyint((f - 1.0) * 8.0);
    if (m == 8) {
        m = 0;
        E += 1;
    }
    if (E > 8 || (E == 8 && m == 7))
        return 0x7E;
    return ((E + 7) << 3) | m;
}

double oracle_e4m3_decode(int b)
{
    int e = (b >> 3) & 15, m = b & 7;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (b & 0x80) ? -v : v;
}

/* ------------------------------------------------------------------ */
/* RMSNorm (the layer normalization the preparation step absorbs)      */
/* ------------------------------------------------------------------ */

/*
 * Sum of q[0..n) as a perfect binary tree over 2^ceil(log2 n) leaves
 * (missing leaves are +0), adjacent pairs at every level, each node one
 * fp32 addition.
 */
float oracle_tree_sum(const float *q, int64_t n)
{
    if (n <= 0)
        return 0.0f;
    int64_t np2 = 1;
    while (np2 < n)
        np2 <<= 1;
    float *a = (float *)calloc((size_t)np2, sizeof(float));
    if (!a)
        abort();
    memcpy(a, q, (size_t)n * sizeof(float));
    for (int64_t w = np2; w > 1; w >>= 1)
        for (int64_t i = 0; i < w / 2; i++)
            a[i] = a[2 * i] + a[2 * i + 1];
    float s = a[0];
    free(a);
    return s;
}

/*
 * The reciprocal RMS of one row: ss = tree sum of fl32(x*x);
 * r = fl32(1 / fl32(sqrt(fl32(fl32(ss / K) + eps)))), with an IEEE square
 * root and division (no reciprocal square root).
 */
float oracle_rms_reciprocal(const uint16_t *x, int64_t k, float eps)
{
    float *q = (float *)malloc((size_t)k * sizeof(float));
    if (!q)
        abort();
    for (int64_t i = 0; i < k; i++) {
        float v = oracle_bf16_to_f32(x[i]);
        q[i] = v * v;
    }
    float ss = oracle_tree_sum(q, k);
    free(q);
    float mean = ss / (float)k;
    float var = mean + eps;
    float s = sqrtf(var);
    return 1.0f / s;
}

/* The normalized row before its rounding to bf16: y = fl32(fl32(x*r)*g). */
void oracle_rmsnorm_scale(const uint16_t *x, const uint16_t *gamma, int64_t k, float r, float *y)
{
    for (int64_t i = 0; i < k; i++) {
        float v = oracle_bf16_to_f32(x[i]);
        float g = oracle_bf16_to_f32(gamma[i]);
        float t = v * r;
        y[i] = t * g;
    }
}

/*
 * RMSNorm of one row: out = bf16(y) with y and r as above.
 * gamma == NULL: no normalization, out = x.
 */
void oracle_rmsnorm_row(const uint16_t *x, const uint16_t *gamma, int64_t k, float eps,
                        uint16_t *out)
{
    if (!gamma) {
        memcpy(out, x, (size_t)k * sizeof(uint16_t));
        return;
    }
    float r = oracle_rms_reciprocal(x, k, eps);
    float *y = (float *)malloc((size_t)k * sizeof(float));
    if (!y)
        abort();
    oracle_rmsnorm_scale(x, gamma, k, r, y);
    for (int64_t i = 0; i < k; i++)
        out[i] = oracle_f32_to_bf16(y[i]);
    free(y);
}

/*
 * Residual add in front of the norm (the fused neighbouring step): the
 * residual stream h and the sublayer output o, both bf16, are added in
 * binary32 and the sum is rounded to bf16, which is what an unfused bf16 add
 * computes; the result is the new residual stream and the input of the
 * RMSNorm.  (The abstract, sentence 5, has the preparation absorb the layer
 * normalization into one operator; in a pre-norm decoder layer the residual
 * add is the step in front of it.)
 */
void oracle_residual_add(const uint16_t *h, const uint16_t *o, int64_t n, uint16_t *x)
{
    for (int64_t i = 0; i < n; i++) {
        float a = oracle_bf16_to_f32(h[i]);
        float b = oracle_bf16_to_f32(o[i]);
        float sum = a + b;
        x[i] = oracle_f32_to_bf16(sum);
    }
}

/*
 * bf16 nearest-even of a double: directly from the double for |v| >= 2^-126
 * (8 significant bits, ties to even; a result of 2^128 or more, and an
 * infinite v, is infinite); below 2^-126, the bf16 subnormal range, through
 * float (the double rounded to float, then to bf16).
 */
uint16_t oracle_f64_to_bf16(double v)
{
    if (isnan(v))                             /* a NaN rounds to a (quiet) NaN */
        return signbit(v) ? 0xFFC0u : 0x7FC0u;
    if (v == 0.0)
        return signbit(v) ? 0x8000u : 0u;
    int e;
    double m = frexp(fabs(v), &e);            /* |v| = m 2^e, m in [0.5, 1) */
    if (e - 1 < -126)
        return oracle_f32_to_bf16((float)v);
    double q = rint(ldexp(m, 8));             /* 8 significant bits, nearest even */
    double r = ldexp(q, e - 8);
    return oracle_f32_to_bf16((float)(signbit(v) ? -r : r));   /* exact: r has 8 bits */
}

/*
 * SiLU(gate) * up in front of the down projection (the other fused
 * neighbouring step): the gate and up halves of the gate+up projection's
 * fp32 output; x = bf16 of g / (1 + exp(-g)) * u evaluated in binary64 and
 * rounded once.  The abstract leaves the MLP's arithmetic open; one rounding
 * of a double evaluation is the plainest reading, and the one a GPU can
 * reproduce exactly without matching this file's exp bit for bit.
 */
void oracle_silu_mul(const float *g, int64_t ld_g, const float *u, int64_t ld_u, int64_t m,
                     int64_t k, uint16_t *x)
{
    for (int64_t r = 0; r < m; r++)
        for (int64_t i = 0; i < k; i++) {
            double gd = (double)g[r * ld_g + i];
            double ud = (double)u[r * ld_u + i];
            double s = gd / (1.0 + exp(-gd));
            double v = s * ud;
            x[r * k + i] = oracle_f64_to_bf16(v);
        }
}

/* ------------------------------------------------------------------ */
/* 2:4 magnitude mask                                                  */
/* ------------------------------------------------------------------ */

/*
 * Keep the two entries of a group of four with the largest magnitude; on
 * equal magnitude the lower index ranks first (+0 and -0 are equal).  The
 * kept indices are returned in increasing order.
 */
void oracle_mask_group(const float v[4], int *i0, int *i1)
{
    int order[4] = {0, 1, 2, 3};
    /* stable insertion sort by magnitude, descending */
    for (int a = 1; a < 4; a++) {
        int cur = order[a];
        int b = a - 1;
        while (b >= 0 && fabsf(v[order[b]]) < fabsf(v[cur])) {
            order[b + 1] = order[b];
            b--;
        }
        order[b + 1] = cur;
    }
    int p = order[0], q = order[1];
    *i0 = p < q ? p : q;
    *i1 = p < q ? q : p;
}

/* ------------------------------------------------------------------ */
/* Block quantizers                                                    */
/* ------------------------------------------------------------------ */

/* MXFP4: one E8M0 scale per block of n values; codes and exact dequant. */
void oracle_mx_block(const float *v, int n, uint8_t *codes, uint8_t *scale_byte, float *deq)
{
    double amax = 0.0;
    for (int i = 0; i < n; i++)
        if (fabs((double)v[i]) > amax)
            amax = fabs((double)v[i]);
    int e = oracle_mx_scale_exp(amax);
    *scale_byte = (uint8_t)(e + 127);
    for (int i = 0; i < n; i++) {
        double t = ldexp((double)v[i], -e);         /* exact */
        int c = oracle_e2m1_encode(t);
        codes[i] = (uint8_t)c;
        deq[i] = (float)ldexp(oracle_e2m1_decode(c), e);  /* exact in fp32 */
    }
}

/*
 * NVFP4-style: E4M3 block scale sb = e4m3(fl32(amax / fl32(6 * s_t))),
 * effective scale S = fl32(e4m3value(sb) * s_t), t = fl32(v / S),
 * dequant fl32(e2m1value * S).  S == 0 gives signed zero codes.
 */
void oracle_nv_block(const float *v, int n, float s_t, uint8_t *codes, uint8_t *scale_byte,
                     float *deq)
{
    float amax = 0.0f;
    for (int i = 0; i < n; i++)
        if (fabsf(v[i]) > amax)
            amax = fabsf(v[i]);
    float d6 = 6.0f * s_t;
    float ratio = amax / d6;
    int sb = oracle_e4m3_encode((double)ratio);
    *scale_byte = (uint8_t)sb;
    float sbv = (float)oracle_e4m3_decode(sb);
    float S = sbv * s_t;
    for (int i = 0; i < n; i++) {
        if (S == 0.0f) {
            codes[i] = signbit(v[i]) ? 8 : 0;
            deq[i] = signbit(v[i]) ? -0.0f : 0.0f;
            continue;
        }
        float t = v[i] / S;
        int c = oracle_e2m1_encode((double)t);
        codes[i] = (uint8_t)c;
        float val = (float)oracle_e2m1_decode(c);
        deq[i] = val * S;
    }
}

static void quant_row(int fmt, const float *v, int64_t k, float s_t, uint8_t *codes,
                      uint8_t *scales, float *deq)
{
    int blk = (fmt == ORACLE_MXFP4) ? 32 : 16;
    for (int64_t b = 0; b < k / blk; b++) {
        if (fmt == ORACLE_MXFP4)
            oracle_mx_block(v + b * blk, blk, codes + b * blk, scales + b, deq + b * blk);
        else
            oracle_nv_block(v + b * blk, blk, s_t, codes + b * blk, scales + b, deq + b * blk);
    }
}

/* Per-tensor fp32 scale of the NVFP4-style format: fl32(amax / 2688), 2688 = 6 * 448. */
float oracle_nv_tensor_scale(float amax)
{
    if (amax == 0.0f)
        return 1.0f;
    return amax / 2688.0f;
}

/* ------------------------------------------------------------------ */
/* Preparation operator                                                */
/* ------------------------------------------------------------------ */

/*
 * Mask, backbone and residual of one normalized row xn_row (k values), with
 * its own work buffers; writes row i of each output array.
 */
static void prepare_row(int fmt, const uint16_t *xn_row, int64_t i, int64_t k, float s_t,
                        uint8_t *meta, uint8_t *s_codes, uint8_t *s_scales, uint8_t *r_codes,
                        uint8_t *r_scales, uint8_t *s_dense)
{
    int blk = (fmt == ORACLE_MXFP4) ? 32 : 16;
    float *xf = (float *)malloc((size_t)k * sizeof(float));
    float *v = (float *)malloc((size_t)k * sizeof(float));
    float *d = (float *)malloc((size_t)k * sizeof(float));
    float *rr = (float *)malloc((size_t)k * sizeof(float));
    uint8_t *cs = (uint8_t *)malloc((size_t)k);
    uint8_t *cr = (uint8_t *)malloc((size_t)k);
    int *keep = (int *)malloc((size_t)k * sizeof(int));
    if (!xf || !v || !d || !rr || !cs || !cr || !keep)
        abort();
    for (int64_t j = 0; j < k; j++)
        xf[j] = oracle_bf16_to_f32(xn_row[j]);
    /* mask */
    for (int64_t g = 0; g < k / 4; g++) {
        int i0, i1;
        oracle_mask_group(xf + 4 * g, &i0, &i1);
        for (int t = 0; t < 4; t++)
            keep[4 * g + t] = (t == i0 || t == i1);
        uint8_t nib = (uint8_t)(i0 | (i1 << 2));
        uint8_t *mb = meta + i * (k / 8) + g / 2;
        if (g % 2 == 0)
            *mb = nib;
        else
            *mb = (uint8_t)(*mb | (nib << 4));
    }
    /* backbone */
    for (int64_t j = 0; j < k; j++)
        v[j] = keep[j] ? xf[j] : 0.0f;
    quant_row(fmt, v, k, s_t, cs, s_scales + i * (k / blk), d);
    for (int64_t g = 0; g < k / 4; g++) {
        int i0 = -1, i1 = -1;
        for (int t = 0; t < 4; t++) {
            if (keep[4 * g + t]) {
                if (i0 < 0) i0 = t; else i1 = t;
            }
        }
        s_codes[i * (k / 4) + g] = (uint8_t)(cs[4 * g + i0] | (cs[4 * g + i1] << 4));
    }
    if (s_dense) {
        for (int64_t j = 0; j < k; j += 2)
            s_dense[i * (k / 2) + j / 2] = (uint8_t)(cs[j] | (cs[j + 1] << 4));
    }
    /* residual against the quantized backbone */
    for (int64_t j = 0; j < k; j++)
        rr[j] = xf[j] - d[j];
    quant_row(fmt, rr, k, s_t, cr, r_scales + i * (k / blk), d);
    for (int64_t j = 0; j < k; j += 2)
        r_codes[i * (k / 2) + j / 2] = (uint8_t)(cr[j] | (cr[j + 1] << 4));
    free(xf); free(v); free(d); free(rr); free(cs); free(cr); free(keep);
}

/*
 * For each row of X [m, k] (bf16, row stride k):
 *   x_n = RMSNorm(x) (or x when gamma == NULL);
 *   2:4 mask on |x_n| per aligned group of four along k;
 *   backbone v = x_n at kept positions, +0 elsewhere, block-quantized;
 *   residual R = fl32(x_n - deq(backbone)), block-quantized.
 * Outputs (row-major, row strides k/8, k/4, k/blk, k/2, k/blk, k/2):
 *   meta     one nibble per group, i0 | i1 << 2; group 2j in the low nibble of byte j
 *   s_codes  one byte per group: code at i0 in the low nibble, code at i1 in the high
 *   s_scales one scale byte per block of the backbone
 *   r_codes  residual codes, two per byte, the lower k in the low nibble
 *   r_scales one scale byte per block of the residual
 *   s_dense  (optional, may be NULL) backbone codes in the dense layout of r_codes
 *   tensor_scale (NVFP4 only) fl32(amax(x_n)/2688), shared by both paths
 * Rows are independent; the row loops may run on several threads (built with
 * OpenMP) without changing any value.  Returns 0, or -1 on a bad argument.
 */
int oracle_prepare(int fmt, const uint16_t *x, int64_t m, int64_t k, const uint16_t *gamma,
                   float eps, uint8_t *meta, uint8_t *s_codes, uint8_t *s_scales,
                   uint8_t *r_codes, uint8_t *r_scales, uint8_t *s_dense, float *tensor_scale)
{
    int blk = (fmt == ORACLE_MXFP4) ? 32 : 16;
    if ((fmt != ORACLE_MXFP4 && fmt != ORACLE_NVFP4) || m < 0 || k <= 0 || k % blk)
        return -1;
    uint16_t *xn = (uint16_t *)malloc((size_t)(m * k + 1) * sizeof(uint16_t));
    if (!xn)
        abort();

    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; i++)
        oracle_rmsnorm_row(x + i * k, gamma, k, eps, xn + i * k);

    float s_t = 1.0f;
    if (fmt == ORACLE_NVFP4) {
        float amax = 0.0f;
        for (int64_t i = 0; i < m * k; i++) {
            float a = fabsf(oracle_bf16_to_f32(xn[i]));
            if (a > amax)
                amax = a;
        }
        s_t = oracle_nv_tensor_scale(amax);
        if (tensor_scale)
            *tensor_scale = s_t;
    }

    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; i++)
        prepare_row(fmt, xn + i * k, i, k, s_t, meta, s_codes, s_scales, r_codes, r_scales,
                    s_dense);
    free(xn);
    return 0;
}

/* Normalized rows only (for tests of the identity deq(backbone) + R = x_n). */
int oracle_normalize(const uint16_t *x, int64_t m, int64_t k, const uint16_t *gamma, float eps,
                     uint16_t *xn)
{
    for (int64_t i = 0; i < m; i++)
        oracle_rmsnorm_row(x + i * k, gamma, k, eps, xn + i * k);
    return 0;
}

/*
 * Residual values in fp32, from the normalized rows and the backbone's
 * exported form (for invariant tests).  Uses the same steps as prepare.
 */
int oracle_residual_f32(int fmt, const uint16_t *xn, int64_t m, int64_t k, float s_t, float *r)
{
    int blk = (fmt == ORACLE_MXFP4) ? 32 : 16;
    if (k % blk)
        return -1;
    float *xf = (float *)malloc((size_t)k * sizeof(float));
    float *v = (float *)malloc((size_t)k * sizeof(float));
    float *d = (float *)malloc((size_t)k * sizeof(float));
    uint8_t *cs = (uint8_t *)malloc((size_t)k);
    uint8_t *sc = (uint8_t *)malloc((size_t)(k / blk));
    if (!xf || !v || !d || !cs || !sc)
        abort();
    for (int64_t i = 0; i < m; i++) {
        for (int64_t j = 0; j < k; j++)
            xf[j] = oracle_bf16_to_f32(xn[i * k + j]);
        for (int64_t g = 0; g < k / 4; g++) {
            int i0, i1;
            oracle_mask_group(xf + 4 * g, &i0, &i1);
            for (int t = 0; t < 4; t++)
                v[4 * g + t] = (t == i0 || t == i1) ? xf[4 * g + t] : 0.0f;
        }
        quant_row(fmt, v, k, s_t, cs, sc, d);
        for (int64_t j = 0; j < k; j++)
            r[i * k + j] = xf[j] - d[j];
    }
    free(xf); free(v); free(d); free(cs); free(sc);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Weight quantization                                                 */
/* ------------------------------------------------------------------ */

/*
 * Each row of W [n, k] (bf16) through the block quantizer, no norm and no
 * mask: codes [n, k/2] (lower k in the low nibble), scales [n, k/blk];
 * NVFP4 uses the weight's own tensor scale fl32(amax(W)/2688).
 */
int oracle_quantize_weight(int fmt, const uint16_t *w, int64_t n, int64_t k, uint8_t *codes,
                           uint8_t *scales, float *tensor_scale)
{
    int blk = (fmt == ORACLE_MXFP4) ? 32 : 16;
    if ((fmt != ORACLE_MXFP4 && fmt != ORACLE_NVFP4) || n < 0 || k <= 0 || k % blk)
        return -1;
    float s_t = 1.0f;
    if (fmt == ORACLE_NVFP4) {
        float amax = 0.0f;
        for (int64_t i = 0; i < n * k; i++) {
            float a = fabsf(oracle_bf16_to_f32(w[i]));
            if (a > amax)
                amax = a;
        }
        s_t = oracle_nv_tensor_scale(amax);
        if (tensor_scale)
            *tensor_scale = s_t;
    }
    float *v = (float *)malloc((size_t)k * sizeof(float));
    float *d = (float *)malloc((size_t)k * sizeof(float));
    uint8_t *c = (uint8_t *)malloc((size_t)k);
    if (!v || !d || !c)
        abort();
    for (int64_t i = 0; i < n; i++) {
        for (int64_t j = 0; j < k; j++)
            v[j] = oracle_bf16_to_f32(w[i * k + j]);
        quant_row(fmt, v, k, s_t, c, scales + i * (k / blk), d);
        for (int64_t j = 0; j < k; j += 2)
            codes[i * (k / 2) + j / 2] = (uint8_t)(c[j] | (c[j + 1] << 4));
    }
    free(v); free(d); free(c);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Dual-path GEMM                                                      */
/* ------------------------------------------------------------------ */

static double scale_value(int fmt, uint8_t b)
{
    /* MXFP4: E8M0 value 2^(b-127); NVFP4: E4M3 block scale (tensor scale applied last) */
    return (fmt == ORACLE_MXFP4) ? ldexp(1.0, (int)b - 127) : oracle_e4m3_decode(b);
}

/* Row i of the backbone, dequantized (without the NVFP4 tensor scale), from its compressed form. */
static void decode_sparse_row(int fmt, const uint8_t *s_codes, const uint8_t *meta,
                              const uint8_t *s_scales, int64_t i, int64_t k, double *out)
{
    int blk = (fmt == ORACLE_MXFP4) ? 32 : 16;
    for (int64_t j = 0; j < k; j++)
        out[j] = 0.0;
    for (int64_t g = 0; g < k / 4; g++) {
        uint8_t mb = meta[i * (k / 8) + g / 2];
        int nib = (g % 2 == 0) ? (mb & 15) : (mb >> 4);
        int i0 = nib & 3, i1 = (nib >> 2) & 3;
        uint8_t cb = s_codes[i * (k / 4) + g];
        double sc = scale_value(fmt, s_scales[i * (k / blk) + (4 * g) / blk]);
        out[4 * g + i0] = oracle_e2m1_decode(cb & 15) * sc;
        out[4 * g + i1] = oracle_e2m1_decode(cb >> 4) * sc;
    }
}

/* Row i of a dense FP4 operand, dequantized (without the NVFP4 tensor scale). */
static void decode_dense_row(int fmt, const uint8_t *codes, const uint8_t *scales, int64_t i,
                             int64_t k, double *out)
{
    int blk = (fmt == ORACLE_MXFP4) ? 32 : 16;
    for (int64_t j = 0; j < k; j++) {
        uint8_t cb = codes[i * (k / 2) + j / 2];
        int c = (j % 2 == 0) ? (cb & 15) : (cb >> 4);
        out[j] = oracle_e2m1_decode(c) * scale_value(fmt, scales[i * (k / blk) + j / blk]);
    }
}

/*
 * Y[i, j] = sum_k ds[i,k] w[j,k] + sum_k dr[i,k] w[j,k] (both sums in k
 * order, one fp64 accumulator, backbone first), NVFP4: times the two tensor
 * scales in fp64; then rounded once to fp32.  Each pair (rows[p], cols[p])
 * gives y[p]; y64 (optional) receives the fp64 value before rounding, and
 * y_abs (optional) the sum of the magnitudes of the same 2k products (with
 * the tensor scales), which bounds the error of any fp32 summation order.
 */
int oracle_dual_gemm_pairs(int fmt, const uint8_t *s_codes, const uint8_t *meta,
                           const uint8_t *s_scales, const uint8_t *r_codes,
                           const uint8_t *r_scales, const float *a_tensor_scale,
                           const uint8_t *w_codes, const uint8_t *w_scales,
                           const float *w_tensor_scale, int64_t k, const int64_t *rows,
                           const int64_t *cols, int64_t count, float *y, double *y64,
                           double *y_abs)
{
    double *ds = (double *)malloc((size_t)k * sizeof(double));
    double *dr = (double *)malloc((size_t)k * sizeof(double));
    double *dw = (double *)malloc((size_t)k * sizeof(double));
    if (!ds || !dr || !dw)
        abort();
    int64_t last_row = -1;
    for (int64_t p = 0; p < count; p++) {
        int64_t i = rows[p], j = cols[p];
        if (i != last_row) {
            decode_sparse_row(fmt, s_codes, meta, s_scales, i, k, ds);
            decode_dense_row(fmt, r_codes, r_scales, i, k, dr);
            last_row = i;
        }
        decode_dense_row(fmt, w_codes, w_scales, j, k, dw);
        double acc = 0.0;
        for (int64_t t = 0; t < k; t++)
            acc += ds[t] * dw[t];
        for (int64_t t = 0; t < k; t++)
            acc += dr[t] * dw[t];
        double mag = 0.0;
        if (y_abs) {
            for (int64_t t = 0; t < k; t++)
                mag += fabs(ds[t] * dw[t]) + fabs(dr[t] * dw[t]);
        }
        if (fmt == ORACLE_NVFP4) {
            acc = acc * (double)*a_tensor_scale * (double)*w_tensor_scale;
            mag = mag * (double)*a_tensor_scale * (double)*w_tensor_scale;
        }
        if (y64)
            y64[p] = acc;
        if (y_abs)
            y_abs[p] = mag;
        y[p] = (float)acc;
    }
    free(ds); free(dr); free(dw);
    return 0;
}

/* Full Y [m, n] (row stride n); same arithmetic as oracle_dual_gemm_pairs,
 * one output row at a time (rows may run on several threads). */
int oracle_dual_gemm(int fmt, const uint8_t *s_codes, const uint8_t *meta,
                     const uint8_t *s_scales, const uint8_t *r_codes, const uint8_t *r_scales,
                     const float *a_tensor_scale, const uint8_t *w_codes,
                     const uint8_t *w_scales, const float *w_tensor_scale, int64_t m, int64_t n,
                     int64_t k, float *y, double *y64, double *y_abs)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; i++) {
        int64_t *rows = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
        int64_t *cols = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
        if (!rows || !cols)
            abort();
        for (int64_t j = 0; j < n; j++) {
            rows[j] = i;
            cols[j] = j;
        }
        oracle_dual_gemm_pairs(fmt, s_codes, meta, s_scales, r_codes, r_scales, a_tensor_scale,
                               w_codes, w_scales, w_tensor_scale, k, rows, cols, n, y + i * n,
                               y64 ? y64 + i * n : NULL, y_abs ? y_abs + i * n : NULL);
        free(rows); free(cols);
    }
    return 0;
}

/* Number of threads the row loops use (1 unless built with OpenMP). */
int oracle_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
