/*
 * fp4kv_oracle.c -- plain, slow CPU oracle for the FP4 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the
 * HIP path: every table below is built from the number-format definitions.
 *
 * What it computes, and where the pages state it:
 *
 *   Quantiser -- "Quantising the KV cache" (numerics-explained), Code section,
 *   the FP4 block quantiser excerpt, and Concept section, paragraph "FP4 with
 *   a fine-grained scale": a row is cut into blocks of 16 consecutive
 *   channels; the block's scale is its largest magnitude divided by 6, rounded
 *   to FP8 E4M3 (round to nearest, ties to even, saturating); a scale that
 *   rounds to zero is replaced by the smallest positive E4M3 subnormal; each
 *   element divided by the scale is rounded to FP4 E2M1 (same rounding) and the
 *   stored value is that E2M1 number times the scale.
 *
 *   Attention -- same page, Code section (the quantised K and V replace the
 *   real ones between the projections and an unchanged attention; Q is not
 *   quantised) and Concept section (every new token reads every cached key
 *   and value).  Attention is written out from its definition in fp64:
 *   z_t = scale * <q, k_t>,  w_t = exp(z_t - max z),  o = sum w_t v_t / sum w_t.
 *
 *   FP8 variant -- same page, Concept section, results table: FP8 E4M3 with
 *   one scale per tensor.  Each element divided by the tensor's scale is
 *   rounded to E4M3 (nearest, ties to even, saturating, as the FP4 encoder
 *   does); the stored value is that E4M3 number times the scale.
 *
 *   Integer formats for the bit-width sweep -- same page, Concept section,
 *   results table (INT8/INT4/INT2 per token, and K per channel with V per
 *   token) and Maths section (cost b + s/g with one FP16 scale per group);
 *   "Week 6 -- FP4 KV Caches and Bounded Replay", Lab section (quantise
 *   synthetic KV at several bit widths and measure the attention output's
 *   error).  The page prints no integer encoder: the symmetric, round-to-
 *   nearest-even rule below is a reading, stated where it is made.
 *
 * Readings where the pages are silent are listed with the functions that
 * make them.  Every arithmetic step here is exact except the exp/sum/divide
 * of the attention, which runs in fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

/* FP4 E2M1 magnitude of a 3-bit code: 2 exponent bits with bias 1, one
 * mantissa bit, a subnormal at exponent 0, no infinity or NaN.
 * Codes 0..7 give 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double fp4kv_oracle_e2m1_value(int code)
{
    int e = (code >> 1) & 3, m = code & 1;
    if (e == 0)
        return 0.5 * m;                         /* subnormal: m * 2^(1-1) * 0.5 */
    return ldexp(1.0 + 0.5 * m, e - 1);
}

/* FP8 E4M3 magnitude of a 7-bit code, OCP "FN" variant (reading: the pages
 * name E4M3 and its smallest subnormal, which fixes bias 7).  4 exponent bits
 * with bias 7, 3 mantissa bits, subnormals at exponent 0; code 0x7F is NaN,
 * so the finite codes are 0..126 and the largest is 0x7E = 448. */
double fp4kv_oracle_e4m3_value(int code)
{
    int e = (code >> 3) & 15, m = code & 7;
    if (e == 0)
        return ldexp((double)m, -9);            /* m/8 * 2^(1-7) */
    return ldexp(1.0 + m / 8.0, e - 7);
}

#define E2M1_MAX_CODE 7
#define E4M3_MAX_CODE 126

/* Round the exact quotient num/den (num >= 0, den > 0) to the nearest finite
 * magnitude of a format, ties to the even code, and saturate anything at or
 * beyond the largest finite magnitude to that magnitude.
 *
 * Reading: the pages call their encoder with mode "rne" and a flag set to
 * true; the flag is read as saturation, as E2M1 has no infinity to overflow
 * into.  The pages divide in double precision before rounding; rounding the
 * exact quotient instead gives the same code for every bf16 input (the
 * quotient is never within a double ulp of a rounding boundary it is not
 * equal to), and keeps this function exact by construction.
 *
 * No division is done: num is compared with value*den, and 2*num with the
 * sum of two neighbouring values times den.  For the operands used here
 * (num a bf16 magnitude, den = 6 or an E4M3 value, values with at most 4
 * significant bits) every product and sum is exact in double. */
static int round_ratio_rne_sat(double num, double den, double (*value)(int), int max_code)
{
    if (num >= value(max_code) * den)
        return max_code;
    int lo = 0;
    while (value(lo + 1) * den <= num)          /* value(lo)*den <= num < value(lo+1)*den */
        lo++;
    double twice = 2.0 * num;
    double mid2 = (value(lo) + value(lo + 1)) * den;
    if (twice < mid2)
        return lo;
    if (twice > mid2)
        return lo + 1;
    return (lo % 2 == 0) ? lo : lo + 1;         /* exactly halfway: the even code */
}

/* E4M3 code of num/den by bisection over the monotone table (same result as
 * round_ratio_rne_sat with the E4M3 table, in 7 steps instead of up to 126):
 * lo = the largest code whose value*den <= num, then the same halfway rule.
 * For den a finite positive fp32 value every product and sum below has at
 * most 24 + 5 significant bits, so it is exact in double. */
static int e4m3_ratio_rne_sat(double num, double den)
{
    if (num >= fp4kv_oracle_e4m3_value(E4M3_MAX_CODE) * den)
        return E4M3_MAX_CODE;
    int lo = 0, hi = E4M3_MAX_CODE;               /* value(lo)*den <= num < value(hi)*den */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (fp4kv_oracle_e4m3_value(mid) * den <= num)
            lo = mid;
        else
            hi = mid;
    }
    double twice = 2.0 * num;
    double mid2 = (fp4kv_oracle_e4m3_value(lo) + fp4kv_oracle_e4m3_value(lo + 1)) * den;
    if (twice < mid2)
        return lo;
    if (twice > mid2)
        return lo + 1;
    return (lo % 2 == 0) ? lo : lo + 1;
}

/* bf16 bit pattern -> its exact value. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------- quantiser */

/* Quantise one block of n (1..16) bf16 values, following the block loop of
 * the page's quantiser excerpt in its order:
 *   amax -> scale code = RNE_sat_E4M3(amax / 6) -> zero scale replaced by the
 *   smallest subnormal -> per element code = RNE_sat_E2M1(|x| / s).
 * Outputs: nib[c] = sign << 3 | magnitude code (reading: the sign of the input
 * is kept, also when the magnitude rounds to zero, as an IEEE conversion
 * does); *scale_code = E4M3 code of s; xhat[c] = +-E2M1(code) * s (may be
 * NULL).  Returns -1 if an input is not finite (inputs must be finite). */
int fp4kv_oracle_quantize_block(const uint16_t *x, int n, uint8_t *nib,
                                uint8_t *scale_code, double *xhat)
{
    double amax = 0.0;
    for (int c = 0; c < n; c++) {
        double v = bf16_value(x[c]);
        if (!isfinite(v))
            return -1;
        if (fabs(v) > amax)
            amax = fabs(v);
    }
    int sc = round_ratio_rne_sat(amax, 6.0, fp4kv_oracle_e4m3_value, E4M3_MAX_CODE);
    if (sc == 0)
        sc = 1;                                  /* the smallest positive E4M3 subnormal, 2^-9 */
    double s = fp4kv_oracle_e4m3_value(sc);
    *scale_code = (uint8_t)sc;
    for (int c = 0; c < n; c++) {
        double v = bf16_value(x[c]);
        int neg = signbit(v) ? 1 : 0;
        int e = round_ratio_rne_sat(fabs(v), s, fp4kv_oracle_e2m1_value, E2M1_MAX_CODE);
        nib[c] = (uint8_t)((neg << 3) | e);
        if (xhat)
            xhat[c] = (neg ? -1.0 : 1.0) * fp4kv_oracle_e2m1_value(e) * s;
    }
    return 0;
}

/* Quantise rows [r0, r1) of a row-major [n_rows][row_len] bf16 array.
 * A row is cut into blocks of 16 consecutive channels; a row length that is
 * not a multiple of 16 leaves a shorter last block (as slicing does).
 * nib: [n_rows][row_len], one code per byte.  scales: [n_rows][n_blocks].
 * xhat: [n_rows][row_len] or NULL. */
static int quantize_row_range(const uint16_t *x, int64_t r0, int64_t r1, int row_len,
                              uint8_t *nib, uint8_t *scales, double *xhat)
{
    int n_blocks = (row_len + 15) / 16;
    for (int64_t r = r0; r < r1; r++) {
        for (int b = 0; b < n_blocks; b++) {
            int c0 = 16 * b;
            int n = row_len - c0 < 16 ? row_len - c0 : 16;
            int rc = fp4kv_oracle_quantize_block(x + r * row_len + c0, n,
                                                 nib + r * row_len + c0,
                                                 scales + r * n_blocks + b,
                                                 xhat ? xhat + r * row_len + c0 : NULL);
            if (rc)
                return rc;
        }
    }
    return 0;
}

typedef struct {
    const uint16_t *x;
    int64_t r0, r1;
    int row_len;
    uint8_t *nib, *scales;
    double *xhat;
    int rc;
} quant_job;

static void *quant_worker(void *arg)
{
    quant_job *j = (quant_job *)arg;
    j->rc = quantize_row_range(j->x, j->r0, j->r1, j->row_len, j->nib, j->scales, j->xhat);
    return NULL;
}

/* Threaded over rows only; each row is quantised exactly as above. */
int fp4kv_oracle_quantize_rows(const uint16_t *x, int64_t n_rows, int row_len,
                               uint8_t *nib, uint8_t *scales, double *xhat, int n_threads)
{
    if (row_len <= 0 || n_rows < 0)
        return -2;
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > 256)
        n_threads = 256;
    if ((int64_t)n_threads > n_rows)
        n_threads = n_rows > 0 ? (int)n_rows : 1;
    if (n_threads == 1)
        return quantize_row_range(x, 0, n_rows, row_len, nib, scales, xhat);
    pthread_t tid[256];
    quant_job job[256];
    int64_t per = (n_rows + n_threads - 1) / n_threads;
    for (int i = 0; i < n_threads; i++) {
        int64_t r0 = i * per, r1 = r0 + per > n_rows ? n_rows : r0 + per;
        if (r0 > r1)
            r0 = r1;
        job[i] = (quant_job){x, r0, r1, row_len, nib, scales, xhat, 0};
        pthread_create(&tid[i], NULL, quant_worker, &job[i]);
    }
    int rc = 0;
    for (int i = 0; i < n_threads; i++) {
        pthread_join(tid[i], NULL);
        if (job[i].rc)
            rc = job[i].rc;
    }
    return rc;
}

/* FP8 E4M3 with one scale per tensor: code = sign << 7 | RNE_sat_E4M3(|x| / s)
 * for n bf16 values and a finite positive fp32 scale s.  Readings: the
 * per-tensor scale is given (the pages leave how it is chosen open; a cache
 * that grows token by token needs it fixed in advance); rounding and
 * saturation as in the FP4 encoder; the sign is kept for magnitudes that
 * round to zero (code 0x80), as for the FP4 nibbles.  Returns -1 if an input
 * is not finite or the scale is not finite and positive. */
int fp4kv_oracle_quantize_fp8(const uint16_t *x, int64_t n, float scale, uint8_t *codes)
{
    double s = (double)scale;
    if (!isfinite(s) || !(s > 0.0))
        return -1;
    for (int64_t i = 0; i < n; i++) {
        double v = bf16_value(x[i]);
        if (!isfinite(v))
            return -1;
        int neg = signbit(v) ? 1 : 0;
        codes[i] = (uint8_t)((neg << 7) | e4m3_ratio_rne_sat(fabs(v), s));
    }
    return 0;
}

/* ------------------------------------------------------------- attention */

/* Dequantised cache value: E2M1(code) * scale, signed by the nibble's sign
 * bit (the page's encoder returns the rounded element times the scale). */
static double fp4_value(uint8_t nib, uint8_t scale_code)
{
    double v = fp4kv_oracle_e2m1_value(nib & 7) * fp4kv_oracle_e4m3_value(scale_code & 0x7F);
    return (nib & 8) ? -v : v;
}

/* Decode attention for the G query heads that share one KV head, over T
 * cached tokens, straight from the definition in fp64.
 *   q:      [G][D] bf16 (not quantised)
 *   k_nib:  token t's codes at k_nib + t*nib_stride, D bytes (one code each)
 *   k_sc:   token t's scale codes at k_sc + t*sc_stride, D/16 bytes
 *   v_nib, v_sc: the same for V
 *   out:    [G][D] fp64.  T == 0 gives zeros (reading: an empty context
 *           attends to nothing).
 * D must be a multiple of 16 here. Returns -1 on bad arguments. */
int fp4kv_oracle_attention(const uint16_t *q, int G, int D, int64_t T,
                           const uint8_t *k_nib, const uint8_t *k_sc,
                           const uint8_t *v_nib, const uint8_t *v_sc,
                           int64_t nib_stride, int64_t sc_stride,
                           double scale, double *out)
{
    if (G < 1 || D < 16 || D % 16 || T < 0)
        return -1;
    for (int i = 0; i < G * D; i++)
        out[i] = 0.0;
    if (T == 0)
        return 0;
    double *z = (double *)malloc(sizeof(double) * (size_t)T);
    double *kv = (double *)malloc(sizeof(double) * (size_t)D);
    if (!z || !kv) {
        free(z);
        free(kv);
        return -3;
    }
    for (int g = 0; g < G; g++) {
        const uint16_t *qg = q + (int64_t)g * D;
        double zmax = -INFINITY;
        for (int64_t t = 0; t < T; t++) {
            double dot = 0.0;
            for (int c = 0; c < D; c++)
                dot += bf16_value(qg[c]) * fp4_value(k_nib[t * nib_stride + c], k_sc[t * sc_stride + c / 16]);
            z[t] = scale * dot;
            if (z[t] > zmax)
                zmax = z[t];
        }
        double wsum = 0.0;
        double *og = out + (int64_t)g * D;
        for (int64_t t = 0; t < T; t++) {
            double w = exp(z[t] - zmax);
            wsum += w;
            for (int c = 0; c < D; c++)
                kv[c] = fp4_value(v_nib[t * nib_stride + c], v_sc[t * sc_stride + c / 16]);
            for (int c = 0; c < D; c++)
                og[c] += w * kv[c];
        }
        for (int c = 0; c < D; c++)
            og[c] /= wsum;
    }
    free(z);
    free(kv);
    return 0;
}

/* Dequantised FP8 value: +-E4M3(code) * scale. */
static double fp8_value(uint8_t code, double scale)
{
    double v = fp4kv_oracle_e4m3_value(code & 0x7F) * scale;
    return (code & 0x80) ? -v : v;
}

/* The same attention for an FP8 cache with per-tensor scales k_scale and
 * v_scale: token t's D codes at k_codes + t*stride (and v_codes). */
int fp4kv_oracle_attention_fp8(const uint16_t *q, int G, int D, int64_t T,
                               const uint8_t *k_codes, const uint8_t *v_codes, int64_t stride,
                               double k_scale, double v_scale, double scale, double *out)
{
    if (G < 1 || D < 1 || T < 0)
        return -1;
    for (int i = 0; i < G * D; i++)
        out[i] = 0.0;
    if (T == 0)
        return 0;
    double *z = (double *)malloc(sizeof(double) * (size_t)T);
    if (!z)
        return -3;
    for (int g = 0; g < G; g++) {
        const uint16_t *qg = q + (int64_t)g * D;
        double zmax = -INFINITY;
        for (int64_t t = 0; t < T; t++) {
            double dot = 0.0;
            for (int c = 0; c < D; c++)
                dot += bf16_value(qg[c]) * fp8_value(k_codes[t * stride + c], k_scale);
            z[t] = scale * dot;
            if (z[t] > zmax)
                zmax = z[t];
        }
        double wsum = 0.0;
        double *og = out + (int64_t)g * D;
        for (int64_t t = 0; t < T; t++) {
            double w = exp(z[t] - zmax);
            wsum += w;
            for (int c = 0; c < D; c++)
                og[c] += w * fp8_value(v_codes[t * stride + c], v_scale);
        }
        for (int c = 0; c < D; c++)
            og[c] /= wsum;
    }
    free(z);
    return 0;
}

typedef struct {
    int64_t i0, i1;
    int G, D;
    const uint16_t *const *q;
    const int64_t *T;
    const uint8_t *const *kc, *const *vc;
    int64_t stride;
    double k_scale, v_scale, scale;
    double *const *out;
    int rc;
} attn8_job;

static void *attn8_worker(void *arg)
{
    attn8_job *j = (attn8_job *)arg;
    for (int64_t i = j->i0; i < j->i1; i++) {
        int rc = fp4kv_oracle_attention_fp8(j->q[i], j->G, j->D, j->T[i], j->kc[i], j->vc[i], j->stride,
                                            j->k_scale, j->v_scale, j->scale, j->out[i]);
        if (rc)
            j->rc = rc;
    }
    return NULL;
}

int fp4kv_oracle_attention_fp8_batch(int64_t n_problems, int G, int D, const uint16_t *const *q,
                                     const int64_t *T, const uint8_t *const *k_codes,
                                     const uint8_t *const *v_codes, int64_t stride, double k_scale,
                                     double v_scale, double scale, double *const *out, int n_threads)
{
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > 256)
        n_threads = 256;
    if ((int64_t)n_threads > n_problems)
        n_threads = n_problems > 0 ? (int)n_problems : 1;
    pthread_t tid[256];
    attn8_job job[256];
    int64_t per = (n_problems + n_threads - 1) / n_threads;
    for (int i = 0; i < n_threads; i++) {
        int64_t i0 = i * per, i1 = i0 + per > n_problems ? n_problems : i0 + per;
        if (i0 > i1)
            i0 = i1;
        job[i] = (attn8_job){i0, i1, G, D, q, T, k_codes, v_codes, stride, k_scale, v_scale, scale, out, 0};
        pthread_create(&tid[i], NULL, attn8_worker, &job[i]);
    }
    int rc = 0;
    for (int i = 0; i < n_threads; i++) {
        pthread_join(tid[i], NULL);
        if (job[i].rc)
            rc = job[i].rc;
    }
    return rc;
}

/* A batch of independent (sequence, KV head) attention problems, run on
 * n_threads threads.  Problem i reads q_ptrs[i] ([G][D]), the code/scale
 * pointers of index i (token stride nib_stride / sc_stride), T[i] tokens,
 * and writes out_ptrs[i] ([G][D]). */
typedef struct {
    int64_t i0, i1;
    int G, D;
    const uint16_t *const *q;
    const int64_t *T;
    const uint8_t *const *kn, *const *ks, *const *vn, *const *vs;
    int64_t nib_stride, sc_stride;
    double scale;
    double *const *out;
    int rc;
} attn_job;

static void *attn_worker(void *arg)
{
    attn_job *j = (attn_job *)arg;
    for (int64_t i = j->i0; i < j->i1; i++) {
        int rc = fp4kv_oracle_attention(j->q[i], j->G, j->D, j->T[i], j->kn[i], j->ks[i],
                                        j->vn[i], j->vs[i], j->nib_stride, j->sc_stride,
                                        j->scale, j->out[i]);
        if (rc)
            j->rc = rc;
    }
    return NULL;
}

int fp4kv_oracle_attention_batch(int64_t n_problems, int G, int D,
                                 const uint16_t *const *q, const int64_t *T,
                                 const uint8_t *const *k_nib, const uint8_t *const *k_sc,
                                 const uint8_t *const *v_nib, const uint8_t *const *v_sc,
                                 int64_t nib_stride, int64_t sc_stride, double scale,
                                 double *const *out, int n_threads)
{
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > 256)
        n_threads = 256;
    if ((int64_t)n_threads > n_problems)
        n_threads = n_problems > 0 ? (int)n_problems : 1;
    pthread_t tid[256];
    attn_job job[256];
    int64_t per = (n_problems + n_threads - 1) / n_threads;
    for (int i = 0; i < n_threads; i++) {
        int64_t i0 = i * per, i1 = i0 + per > n_problems ? n_problems : i0 + per;
        if (i0 > i1)
            i0 = i1;
        job[i] = (attn_job){i0, i1, G, D, q, T, k_nib, k_sc, v_nib, v_sc,
                            nib_stride, sc_stride, scale, out, 0};
        pthread_create(&tid[i], NULL, attn_worker, &job[i]);
    }
    int rc = 0;
    for (int i = 0; i < n_threads; i++) {
        pthread_join(tid[i], NULL);
        if (job[i].rc)
            rc = job[i].rc;
    }
    return rc;
}

/* ------------------------------------------------ integer formats (sweep) */

/* IEEE binary16 magnitude of a 15-bit code: 5 exponent bits with bias 15,
 * 10 mantissa bits, subnormals at exponent 0; codes 0..0x7BFF are finite and
 * 0x7BFF = 65504 is the largest. */
double fp4kv_oracle_fp16_value(int code)
{
    int e = (code >> 10) & 31, m = code & 1023;
    if (e == 0)
        return ldexp((double)m, -24);           /* m/1024 * 2^(1-15) */
    return ldexp(1.0 + m / 1024.0, e - 15);
}

#define FP16_MAX_CODE 0x7BFF

/* fp16 code of num/den (num >= 0, den a small positive integer), nearest,
 * ties to the even code, saturating at 65504 -- the E4M3 bisection again over
 * the binary16 table.  value*den has at most 11 + 7 significant bits and the
 * sum of two neighbours times den at most 12 + 7, so both are exact. */
static int fp16_ratio_rne_sat(double num, double den)
{
    if (num >= fp4kv_oracle_fp16_value(FP16_MAX_CODE) * den)
        return FP16_MAX_CODE;
    int lo = 0, hi = FP16_MAX_CODE;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (fp4kv_oracle_fp16_value(mid) * den <= num)
            lo = mid;
        else
            hi = mid;
    }
    double twice = 2.0 * num;
    double mid2 = (fp4kv_oracle_fp16_value(lo) + fp4kv_oracle_fp16_value(lo + 1)) * den;
    if (twice < mid2)
        return lo;
    if (twice > mid2)
        return lo + 1;
    return (lo % 2 == 0) ? lo : lo + 1;
}

/* Nearest integer to num/den (num >= 0, den > 0), ties to the even integer,
 * capped at cap.  Only integers up to cap + 1 are tried, so every product
 * k*den (k <= 128, den an fp16 value) is exact in double. */
static int int_ratio_rne_cap(double num, double den, int cap)
{
    if (num >= (cap + 0.5) * den)               /* at or past the last halfway point */
        return cap;
    int k = 0;                                  /* k*den <= num < (k+1)*den */
    while ((k + 1) * den <= num)
        k++;
    double twice = 2.0 * num;
    double mid2 = (2.0 * k + 1.0) * den;
    if (twice < mid2)
        return k;
    if (twice > mid2)
        return k + 1;
    return (k % 2 == 0) ? k : k + 1;
}

/* Symmetric integer quantisation of bits-bit numbers (bits 2..8) with one
 * fp16 scale per group -- the INT rows of "Quantising the KV cache", Concept
 * section, results table, at the cost b + 16/g of its Maths section.
 *
 * The page prints no integer encoder, so each step is a reading, the
 * plainest the page supports:
 *   qmax = 2^(bits-1) - 1 (a symmetric range: the cost formula counts one
 *   16-bit number per group, a scale and no zero point);
 *   scale code = fp16 nearest-even, saturating, of amax / qmax; a scale that
 *   rounds to zero becomes the smallest fp16 subnormal (as the page's FP4
 *   encoder does with its E4M3 scale);
 *   code = sign(x) * nearest-even integer of |x| / s, capped at qmax
 *   (the same rounding mode as the page's encoder);
 *   the stored value is code * s.
 *
 * Group i's element j is x[i*group_stride + j*elem_stride]; its code goes to
 * the same index of codes, its scale code to scale_codes[i].  A group is one
 * token's channels of one head (per token, elem_stride 1) or one channel of
 * one head across the tokens (per channel, elem_stride = heads * head_dim).
 * Returns -1 on bad arguments or a non-finite input. */
int fp4kv_oracle_quantize_int(const uint16_t *x, int64_t n_groups, int64_t group_len,
                              int64_t group_stride, int64_t elem_stride, int bits,
                              int8_t *codes, uint16_t *scale_codes)
{
    if (bits < 2 || bits > 8 || n_groups < 0 || group_len < 1)
        return -1;
    const int qmax = (1 << (bits - 1)) - 1;
    for (int64_t i = 0; i < n_groups; i++) {
        const int64_t base = i * group_stride;
        double amax = 0.0;
        for (int64_t j = 0; j < group_len; j++) {
            double v = bf16_value(x[base + j * elem_stride]);
            if (!isfinite(v))
                return -1;
            if (fabs(v) > amax)
                amax = fabs(v);
        }
        int sc = fp16_ratio_rne_sat(amax, (double)qmax);
        if (sc == 0)
            sc = 1;
        scale_codes[i] = (uint16_t)sc;
        const double s = fp4kv_oracle_fp16_value(sc);
        for (int64_t j = 0; j < group_len; j++) {
            double v = bf16_value(x[base + j * elem_stride]);
            int c = int_ratio_rne_cap(fabs(v), s, qmax);
            codes[base + j * elem_stride] = (int8_t)(signbit(v) ? -c : c);
        }
    }
    return 0;
}

/* FP8 E4M3 codes with one fp16 scale per group: the finer FP8 scale
 * granularities ("KV Cache Quantisation", Common questions: sweep FP8 scale
 * granularities when checking quality), over the two groupings of "Quantising
 * the KV cache", Concept section (one token's channels, or one channel across
 * the tokens).  The pages give no encoder for them; the reading follows the
 * page's FP4 encoder with E4M3 elements and the integer rows' fp16 scale:
 *   scale code = fp16 nearest-even, saturating, of amax / 448 (448 the
 *   largest finite E4M3 magnitude, as the FP4 encoder divides by E2M1's
 *   largest, 6); a scale that rounds to zero becomes the smallest fp16
 *   subnormal;
 *   code = sign bit | E4M3 nearest-even, saturating, of |x| / s (the sign is
 *   kept for magnitudes that round to zero, as in the per-tensor encoder);
 *   the stored value is +-E4M3(code) * s.
 * Groups and strides as in fp4kv_oracle_quantize_int.  Every product below is
 * exact in double: amax / 448 is decided on fp16 values (11 bits) times 448
 * (3 bits), |x| / s on E4M3 values (4 bits) times an fp16 s.  Returns -1 on
 * bad arguments or a non-finite input. */
int fp4kv_oracle_quantize_fp8_groups(const uint16_t *x, int64_t n_groups, int64_t group_len,
                                     int64_t group_stride, int64_t elem_stride,
                                     uint8_t *codes, uint16_t *scale_codes)
{
    if (n_groups < 0 || group_len < 1)
        return -1;
    const double top = fp4kv_oracle_e4m3_value(E4M3_MAX_CODE);
    for (int64_t i = 0; i < n_groups; i++) {
        const int64_t base = i * group_stride;
        double amax = 0.0;
        for (int64_t j = 0; j < group_len; j++) {
            double v = bf16_value(x[base + j * elem_stride]);
            if (!isfinite(v))
                return -1;
            if (fabs(v) > amax)
                amax = fabs(v);
        }
        int sc = fp16_ratio_rne_sat(amax, top);
        if (sc == 0)
            sc = 1;
        scale_codes[i] = (uint16_t)sc;
        const double s = fp4kv_oracle_fp16_value(sc);
        for (int64_t j = 0; j < group_len; j++) {
            double v = bf16_value(x[base + j * elem_stride]);
            codes[base + j * elem_stride] = (uint8_t)(((signbit(v) ? 1 : 0) << 7) | e4m3_ratio_rne_sat(fabs(v), s));
        }
    }
    return 0;
}

/* Attention of G bf16 query rows over T tokens whose K and V are given as
 * exact values (fp64, token t's D values at k + t*stride): the same fp64
 * definition as above, for any format once it is dequantised, and for the
 * unquantised bf16 cache itself. */
int fp4kv_oracle_attention_values(const uint16_t *q, int G, int D, int64_t T,
                                  const double *k, const double *v, int64_t stride,
                                  double scale, double *out)
{
    if (G < 1 || D < 1 || T < 0)
        return -1;
    for (int i = 0; i < G * D; i++)
        out[i] = 0.0;
    if (T == 0)
        return 0;
    double *z = (double *)malloc(sizeof(double) * (size_t)T);
    if (!z)
        return -3;
    for (int g = 0; g < G; g++) {
        const uint16_t *qg = q + (int64_t)g * D;
        double zmax = -INFINITY;
        for (int64_t t = 0; t < T; t++) {
            double dot = 0.0;
            for (int c = 0; c < D; c++)
                dot += bf16_value(qg[c]) * k[t * stride + c];
            z[t] = scale * dot;
            if (z[t] > zmax)
                zmax = z[t];
        }
        double wsum = 0.0;
        double *og = out + (int64_t)g * D;
        for (int64_t t = 0; t < T; t++) {
            double w = exp(z[t] - zmax);
            wsum += w;
            for (int c = 0; c < D; c++)
                og[c] += w * v[t * stride + c];
        }
        for (int c = 0; c < D; c++)
            og[c] /= wsum;
    }
    free(z);
    return 0;
}

typedef struct {
    int64_t i0, i1;
    int G, D;
    const uint16_t *const *q;
    const int64_t *T;
    const double *const *k, *const *v;
    int64_t stride;
    double scale;
    double *const *out;
    int rc;
} attnv_job;

static void *attnv_worker(void *arg)
{
    attnv_job *j = (attnv_job *)arg;
    for (int64_t i = j->i0; i < j->i1; i++) {
        int rc = fp4kv_oracle_attention_values(j->q[i], j->G, j->D, j->T[i], j->k[i], j->v[i],
                                               j->stride, j->scale, j->out[i]);
        if (rc)
            j->rc = rc;
    }
    return NULL;
}

int fp4kv_oracle_attention_values_batch(int64_t n_problems, int G, int D, const uint16_t *const *q,
                                        const int64_t *T, const double *const *k,
                                        const double *const *v, int64_t stride, double scale,
                                        double *const *out, int n_threads)
{
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > 256)
        n_threads = 256;
    if ((int64_t)n_threads > n_problems)
        n_threads = n_problems > 0 ? (int)n_problems : 1;
    pthread_t tid[256];
    attnv_job job[256];
    int64_t per = (n_problems + n_threads - 1) / n_threads;
    for (int i = 0; i < n_threads; i++) {
        int64_t i0 = i * per, i1 = i0 + per > n_problems ? n_problems : i0 + per;
        if (i0 > i1)
            i0 = i1;
        job[i] = (attnv_job){i0, i1, G, D, q, T, k, v, stride, scale, out, 0};
        pthread_create(&tid[i], NULL, attnv_worker, &job[i]);
    }
    int rc = 0;
    for (int i = 0; i < n_threads; i++) {
        pthread_join(tid[i], NULL);
        if (job[i].rc)
            rc = job[i].rc;
    }
    return rc;
}
