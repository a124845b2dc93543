/*
 * fp4kv_int.h -- KV formats of the bit-width sweep, on MI355X (gfx950):
 * symmetric INT8 / INT4 / INT2 codes and FP8 E4M3 codes with one fp16 scale
 * per token or per channel, the unquantised bf16 cache beside them, and
 * decode attention over any of them.
 *
 * ("Quantising the KV cache", numerics-explained: Concept section, results
 * table -- INT8, INT4 and INT2 per token, and INT4 / INT2 with K per channel
 * and V per token, next to FP16, FP8 and FP4; Maths section -- one FP16 scale
 * per group, b + 16/g bits per number.  "Week 6 -- FP4 KV Caches and Bounded
 * Replay", Lab section -- quantise synthetic KV at several bit widths and
 * measure the attention output's error.  "KV Cache Quantisation", Common
 * questions -- sweep the FP8 scale granularities too.)
 *
 * The page gives no integer encoder.  The one here is symmetric:
 *   qmax  = 2^(bits-1) - 1                      (127, 7, 1)
 *   scale = fp16 round-to-nearest-even of amax / qmax, saturating at 65504;
 *           a scale that rounds to 0 becomes the smallest fp16 subnormal
 *           2^-24 (as the page's FP4 encoder does with its E4M3 scale)
 *   code  = sign(x) * round-to-nearest-even(|x| / scale), capped at qmax
 *   value = code * scale                         (exact in fp32)
 * The FP8 format (bits = FP4KV_INT_FP8_E4M3) takes the page's FP4 encoder
 * with E4M3 elements and the same fp16 scales:
 *   scale = fp16 round-to-nearest-even of amax / 448, saturating, zero ->
 *           2^-24 as above (448 is the largest finite E4M3 magnitude)
 *   code  = sign bit | E4M3 (OCP FN) round-to-nearest-even of |x| / scale,
 *           saturating at 448 (code 0x7E); the sign is kept for magnitudes
 *           that round to zero
 *   value = +-E4M3(code) * scale                 (exact in fp32)
 * where amax is the group's largest magnitude and a group is
 *   per token:   one token's D channels of one KV head;
 *   per channel: one channel of one KV head across the sequence's T tokens.
 *
 * Layout (every sequence holds the same T tokens):
 *   input x   bf16 [B][T][H][D]                  (token-major, as produced)
 *   codes     [B][H][T][D * bits / 8] bytes      (head-major rows); within a
 *             row, bits 8: one two's-complement byte per channel; bits 4:
 *             channel 2i in the low nibble of byte i, 2i+1 in the high;
 *             bits 2: channel 4i+j in bits 2j..2j+1 of byte i (two's
 *             complement fields); FP8: one E4M3 byte per channel; bits 16:
 *             the bf16 values themselves
 *   scales    fp16 bit patterns, per token [B][H][T], per channel [B][H][D];
 *             none for bits 16.
 *
 * Conventions are those of fp4kv.h: device pointers where marked, the
 * caller owns every buffer, work is enqueued on `stream`, host-visible
 * arguments are checked before any HIP call, inputs must be finite.
 */
#ifndef FP4KV_INT_H
#define FP4KV_INT_H

#include <stdint.h>

#include "fp4kv.h"

#ifdef __cplusplus
extern "C" {
#endif

enum fp4kv_int_granularity {
    FP4KV_INT_PER_TOKEN = 0,              /* one scale per (sequence, token, KV head) */
    FP4KV_INT_PER_CHANNEL = 1             /* one scale per (sequence, KV head, channel) */
};

/* The `bits` argument below names the element format: 2, 4 or 8 (symmetric
 * integers), 16 (bf16, unquantised) or this value (FP8 E4M3 codes, one byte
 * each, with the fp16 scales above). */
enum { FP4KV_INT_FP8_E4M3 = 0x108 };

/* Shape of a K or V tensor in one of these formats. */
typedef struct fp4kv_int_dims {
    int32_t batch;                        /* B >= 0 */
    int32_t tokens;                       /* T >= 0, the same for every sequence */
    int32_t num_kv_heads;                 /* H >= 1 */
    int32_t head_dim;                     /* D: 64 or 128 */
} fp4kv_int_dims;

/* Bytes of the code and scale buffers for one tensor.  Host only.
 * bits: 2, 4, 8, FP4KV_INT_FP8_E4M3, or 16 (the unquantised bf16 cache;
 * scale_bytes 0).
 * Errors: INVALID_ARGUMENT (null pointer, negative size, H < 1, unknown
 * granularity, bits not one of the five), UNSUPPORTED (D not 64 or 128). */
FP4KV_API int fp4kv_int_sizes(const fp4kv_int_dims *dims, int32_t bits, int32_t granularity,
                              int64_t *code_bytes_out, int64_t *scale_bytes_out);

/* Quantise one tensor (K or V) of B sequences of T tokens.
 *   x       device bf16 [B][T][H][D], 16-B aligned.
 *   codes   device, code_bytes from fp4kv_int_sizes, 16-B aligned.
 *   scales  device, scale_bytes, 16-B aligned (NULL allowed for bits 16).
 * Per channel, the scales are computed first (one pass over the tensor) and
 * the codes in a second pass; per token, one pass.  B, T = 0 is a no-op.
 * Errors: as fp4kv_int_sizes, plus INVALID_ARGUMENT for a null pointer
 * where data is due, MISALIGNED, HIP. */
FP4KV_API int fp4kv_int_quantize(const fp4kv_int_dims *dims, int32_t bits, int32_t granularity,
                                 const void *x, void *codes, void *scales, void *stream);

/* Split count and workspace bytes for fp4kv_int_decode_attention.  Host
 * only.  The T tokens are cut into S splits of whole 256-token chunks; one
 * workgroup attends over each (sequence, KV head, split) and leaves one
 * partial per query head.  num_splits > 0 asks for S (clamped to the chunk
 * count, at least 1); 0 lets the library choose about 2048 workgroups in
 * total.  Workspace: o fp32 [B][S][num_q_heads][D] at byte 0, then
 * (m, l) fp32 pairs [B][S][num_q_heads] at round_up(o bytes, 256).
 * Errors: INVALID_ARGUMENT (null pointer, bad dims, num_q_heads < 1 or not
 * a multiple of H, num_splits < 0), UNSUPPORTED (more than
 * FP4KV_MAX_GROUP query heads per KV head, D not 64 or 128). */
FP4KV_API int fp4kv_int_decode_plan(const fp4kv_int_dims *dims, int32_t num_q_heads, int32_t num_splits,
                                    int32_t *splits_out, int64_t *workspace_bytes_out);

/* Decode attention, one query token per sequence, over K and V stored in
 * one of the formats above (both tensors with the same bits; each with its
 * own granularity).  For sequence b and query head h (KV head h / G):
 *   out[b][h] = sum_t softmax_t(softmax_scale * q[b][h] . K^[t]) V^[t]
 * with K^, V^ the stored values (code * scale, +-E4M3(code) * scale for
 * FP8, or bf16 for bits 16).  The
 * scales are applied where they factor out: a per-token K scale multiplies
 * the token's score, a per-channel K scale multiplies q, a per-token V scale
 * multiplies the token's weight, a per-channel V scale multiplies the
 * output.  Both products run on the matrix cores with bf16 operands that
 * hold the stored values exactly (the query exactly too; times per-channel
 * K scales, as three bf16 terms) and the weights as two bf16 terms (~2^-15
 * relative); accumulation is fp32.  The splits are merged by the combine
 * kernel of fp4kv_decode_combine.
 *   q           device bf16 [B][num_q_heads][D], 16-B aligned.
 *   k_*, v_*    as written by fp4kv_int_quantize with these dims.
 *   workspace   device, 256-B aligned, >= the plan's bytes; contents on
 *               entry do not matter.
 *   out         device fp32 [B][num_q_heads][D], 16-B aligned.  T = 0 gives
 *               zero rows.
 * Errors: as for the plan, plus INVALID_ARGUMENT (unknown bits, bad
 * granularity, null pointer), MISALIGNED, WORKSPACE_TOO_SMALL, HIP. */
FP4KV_API int fp4kv_int_decode_attention(const fp4kv_int_dims *dims, int32_t bits,
                                         int32_t k_granularity, int32_t v_granularity,
                                         const void *k_codes, const void *k_scales,
                                         const void *v_codes, const void *v_scales,
                                         const void *q, int32_t num_q_heads, float softmax_scale,
                                         int32_t num_splits, void *workspace, int64_t workspace_bytes,
                                         float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4KV_INT_H */
