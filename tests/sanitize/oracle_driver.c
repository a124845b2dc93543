/* Drives every function the C oracle (oracle/fp4kv_oracle.c) exports, on
 * small inputs and with several threads, under AddressSanitizer and
 * UndefinedBehaviorSanitizer: whole-range value tables, block and row
 * quantisers (all bf16 values, zeros, negatives), FP8, integer and grouped
 * FP8 quantisers at both granularities, and the attention functions, single
 * and batched (threaded), including empty contexts and bad arguments.
 * Prints "ok" and exits 0 when every expectation holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double fp4kv_oracle_e2m1_value(int code);
double fp4kv_oracle_e4m3_value(int code);
double fp4kv_oracle_fp16_value(int code);
int fp4kv_oracle_quantize_block(const uint16_t *x, int n, uint8_t *nib, uint8_t *scale_code, double *xhat);
int fp4kv_oracle_quantize_rows(const uint16_t *x, int64_t n_rows, int row_len, uint8_t *nib, uint8_t *scales,
                               double *xhat, int n_threads);
int fp4kv_oracle_quantize_fp8(const uint16_t *x, int64_t n, float scale, uint8_t *codes);
int fp4kv_oracle_attention(const uint16_t *q, int G, int D, int64_t T, const uint8_t *k_nib, const uint8_t *k_sc,
                           const uint8_t *v_nib, const uint8_t *v_sc, int64_t nib_stride, int64_t sc_stride,
                           double scale, double *out);
int fp4kv_oracle_attention_batch(int64_t n_problems, int G, int D, const uint16_t *const *q, const int64_t *T,
                                 const uint8_t *const *k_nib, const uint8_t *const *k_sc,
                                 const uint8_t *const *v_nib, const uint8_t *const *v_sc, int64_t nib_stride,
                                 int64_t sc_stride, double scale, double *const *out, int n_threads);
int fp4kv_oracle_attention_fp8(const uint16_t *q, int G, int D, int64_t T, const uint8_t *k_codes,
                               const uint8_t *v_codes, int64_t stride, double k_scale, double v_scale, double scale,
                               double *out);
int fp4kv_oracle_attention_fp8_batch(int64_t n_problems, int G, int D, const uint16_t *const *q, const int64_t *T,
                                     const uint8_t *const *k_codes, const uint8_t *const *v_codes, int64_t stride,
                                     double k_scale, double v_scale, double scale, double *const *out,
                                     int n_threads);
int fp4kv_oracle_quantize_int(const uint16_t *x, int64_t n_groups, int64_t group_len, int64_t group_stride,
                              int64_t elem_stride, int bits, int8_t *codes, uint16_t *scale_codes);
int fp4kv_oracle_quantize_fp8_groups(const uint16_t *x, int64_t n_groups, int64_t group_len, int64_t group_stride,
                                     int64_t elem_stride, uint8_t *codes, uint16_t *scale_codes);
int fp4kv_oracle_attention_values(const uint16_t *q, int G, int D, int64_t T, const double *k, const double *v,
                                  int64_t stride, double scale, double *out);
int fp4kv_oracle_attention_values_batch(int64_t n_problems, int G, int D, const uint16_t *const *q,
                                        const int64_t *T, const double *const *k, const double *const *v,
                                        int64_t stride, double scale, double *const *out, int n_threads);

static int failures = 0;
#define EXPECT(c)                                                                  \
    do {                                                                           \
        if (!(c)) {                                                                \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                            \
        }                                                                          \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint16_t rand_bf16(int max_exp)   /* finite bf16 with |x| < 2^max_exp */
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    const uint16_t e = (uint16_t)((rng >> 8) % (unsigned)(127 + max_exp));
    return (uint16_t)(((rng >> 40) & 0x8000u) | (e << 7) | ((rng >> 20) & 0x7Fu));
}

static void tables(void)
{
    for (int c = 0; c < 16; c++)
        EXPECT(isfinite(fp4kv_oracle_e2m1_value(c)));
    for (int c = 0; c < 256; c++)
        (void)fp4kv_oracle_e4m3_value(c);
    for (int c = 0; c < 65536; c += 7)
        (void)fp4kv_oracle_fp16_value(c);
}

static void quantisers(void)
{
    /* every finite bf16 magnitude as a block maximum, both signs */
    uint16_t blk[16];
    uint8_t nib[16], sc;
    double xhat[16];
    for (uint32_t a = 0; a < 0x7F80u; a++) {
        memset(blk, 0, sizeof blk);
        blk[a % 16] = (uint16_t)(a | ((a & 1u) << 15));
        EXPECT(fp4kv_oracle_quantize_block(blk, 16, nib, &sc, xhat) == 0);
    }
    blk[0] = 0x7F80; /* infinity */
    EXPECT(fp4kv_oracle_quantize_block(blk, 16, nib, &sc, NULL) == -1);
    /* rows, threaded */
    const int64_t rows = 777;
    const int len = 128;
    uint16_t *x = malloc(sizeof(uint16_t) * rows * len);
    uint8_t *rn = malloc((size_t)rows * len), *rs = malloc((size_t)rows * len / 16);
    double *rx = malloc(sizeof(double) * rows * len);
    for (int64_t i = 0; i < rows * len; i++)
        x[i] = rand_bf16(20);
    EXPECT(fp4kv_oracle_quantize_rows(x, rows, len, rn, rs, rx, 5) == 0);
    EXPECT(fp4kv_oracle_quantize_rows(x, rows, len, rn, rs, NULL, 1) == 0);
    EXPECT(fp4kv_oracle_quantize_rows(x, rows, 0, rn, rs, NULL, 1) != 0);
    /* FP8 over every bf16 value */
    uint16_t *all = malloc(sizeof(uint16_t) * 65536);
    uint8_t *codes = malloc(65536);
    int64_t n = 0;
    for (uint32_t b = 0; b < 65536; b++)
        if ((b & 0x7F80u) != 0x7F80u)
            all[n++] = (uint16_t)b;
    EXPECT(fp4kv_oracle_quantize_fp8(all, n, 0.25f, codes) == 0);
    EXPECT(fp4kv_oracle_quantize_fp8(all, n, -1.0f, codes) != 0);
    /* integer and grouped FP8: per token (elem stride 1) and per channel */
    int8_t *ic = malloc((size_t)rows * len);
    uint16_t *isc = malloc(sizeof(uint16_t) * rows * len);
    for (int bits = 2; bits <= 8; bits += 2) {
        EXPECT(fp4kv_oracle_quantize_int(x, rows, len, len, 1, bits, ic, isc) == 0);
        EXPECT(fp4kv_oracle_quantize_int(x, len, rows, 1, len, bits, ic, isc) == 0);
    }
    EXPECT(fp4kv_oracle_quantize_int(x, rows, len, len, 1, 9, ic, isc) != 0);
    EXPECT(fp4kv_oracle_quantize_fp8_groups(x, rows, len, len, 1, (uint8_t *)ic, isc) == 0);
    EXPECT(fp4kv_oracle_quantize_fp8_groups(x, len, rows, 1, len, (uint8_t *)ic, isc) == 0);
    free(x); free(rn); free(rs); free(rx); free(all); free(codes); free(ic); free(isc);
}

static void attention(void)
{
    enum { G = 4, D = 128, P = 6 };
    int64_t T[P] = {0, 1, 63, 64, 65, 300};
    uint16_t *q[P];
    uint8_t *kn[P], *ks[P], *vn[P], *vs[P], *kc[P], *vc[P];
    double *kv[P], *vv[P], *out[P];
    for (int p = 0; p < P; p++) {
        const int64_t t = T[p] ? T[p] : 1;
        q[p] = malloc(sizeof(uint16_t) * G * D);
        for (int i = 0; i < G * D; i++)
            q[p][i] = rand_bf16(3);
        uint16_t *rows = malloc(sizeof(uint16_t) * t * D);
        for (int64_t i = 0; i < t * D; i++)
            rows[i] = rand_bf16(4);
        kn[p] = malloc((size_t)t * D); ks[p] = malloc((size_t)t * D / 16);
        vn[p] = malloc((size_t)t * D); vs[p] = malloc((size_t)t * D / 16);
        kc[p] = malloc((size_t)t * D); vc[p] = malloc((size_t)t * D);
        kv[p] = malloc(sizeof(double) * t * D); vv[p] = malloc(sizeof(double) * t * D);
        out[p] = malloc(sizeof(double) * G * D);
        EXPECT(fp4kv_oracle_quantize_rows(rows, t, D, kn[p], ks[p], kv[p], 2) == 0);
        EXPECT(fp4kv_oracle_quantize_rows(rows, t, D, vn[p], vs[p], vv[p], 2) == 0);
        EXPECT(fp4kv_oracle_quantize_fp8(rows, t * D, 0.05f, kc[p]) == 0);
        EXPECT(fp4kv_oracle_quantize_fp8(rows, t * D, 0.05f, vc[p]) == 0);
        free(rows);
        EXPECT(fp4kv_oracle_attention(q[p], G, D, T[p], kn[p], ks[p], vn[p], vs[p], D, D / 16, 0.088, out[p]) == 0);
        EXPECT(fp4kv_oracle_attention_fp8(q[p], G, D, T[p], kc[p], vc[p], D, 0.05, 0.05, 0.088, out[p]) == 0);
        EXPECT(fp4kv_oracle_attention_values(q[p], G, D, T[p], kv[p], vv[p], D, 0.088, out[p]) == 0);
    }
    EXPECT(fp4kv_oracle_attention_batch(P, G, D, (const uint16_t *const *)q, T, (const uint8_t *const *)kn,
                                        (const uint8_t *const *)ks, (const uint8_t *const *)vn,
                                        (const uint8_t *const *)vs, D, D / 16, 0.088, out, 4) == 0);
    EXPECT(fp4kv_oracle_attention_fp8_batch(P, G, D, (const uint16_t *const *)q, T, (const uint8_t *const *)kc,
                                            (const uint8_t *const *)vc, D, 0.05, 0.05, 0.088, out, 3) == 0);
    EXPECT(fp4kv_oracle_attention_values_batch(P, G, D, (const uint16_t *const *)q, T, (const double *const *)kv,
                                               (const double *const *)vv, D, 0.088, out, 6) == 0);
    EXPECT(fp4kv_oracle_attention(q[0], 0, D, 5, kn[5], ks[5], vn[5], vs[5], D, D / 16, 0.088, out[0]) != 0);
    EXPECT(fp4kv_oracle_attention(q[0], G, 24, 5, kn[5], ks[5], vn[5], vs[5], D, D / 16, 0.088, out[0]) != 0);
    EXPECT(fp4kv_oracle_attention_fp8(q[0], G, D, -1, kc[5], vc[5], D, 0.05, 0.05, 0.088, out[0]) != 0);
    for (int p = 0; p < P; p++) {
        free(q[p]); free(kn[p]); free(ks[p]); free(vn[p]); free(vs[p]); free(kc[p]); free(vc[p]);
        free(kv[p]); free(vv[p]); free(out[p]);
    }
}

int main(void)
{
    tables();
    quantisers();
    attention();
    if (failures) {
        fprintf(stderr, "%d expectations failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
