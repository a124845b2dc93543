/*
 * fp4kv.h -- C ABI of the FP4 KV-cache library for AMD MI355X (gfx950).
 *
 * The cache stores every past token's keys and values with FP4 E2M1
 * elements and one FP8 E4M3 (OCP "FN") scale per 16 consecutive channels of
 * a token's row: 4 + 8/16 = 4.5 bits per number, 28.125% of an FP16 cache.
 * ("Quantising the KV cache", numerics-explained: Concept section, paragraph
 * on FP4 with a fine-grained scale; Maths section for the cost; Code section
 * for the block quantiser.)
 *
 * Calls:
 *   fp4kv_cache_layout      sizes and lays out a paged cache (host only).
 *   fp4kv_quantize_append   quantises new tokens' K and V rows into the cache.
 *   fp4kv_decode_plan       chooses the split count and workspace size.
 *   fp4kv_decode_attention  split-K decode attention over the packed cache,
 *                           dequantising on the fly.
 *   fp4kv_decode_attention_noalloc
 *                           the same with a static workspace, for callers
 *                           that cannot allocate.
 *   fp4kv_decode_split,     its two halves: per-split partial results, and
 *   fp4kv_decode_combine    their merge.
 *   fp4kv_decode_append_attention, fp4kv_decode_append_split
 *                           a decode step that first stores each sequence's
 *                           new token (fused into the decode kernel).
 *   fp4kv_decode_multi_attention
 *                           several query tokens per sequence, causal.
 *   fp4kv_decode_window_plan, fp4kv_decode_window_attention
 *                           the same with a sliding window.
 *   fp4kv_decode_with_options
 *                           any of the above with an explicit kernel and
 *                           merge choice (tests, measurements).
 *   fp4kv_status_string     text of a status code.
 *
 * Conventions for every call:
 *   - Pointers marked "device" are HIP device memory; all others are host.
 *   - The caller owns every buffer.  The library allocates nothing, keeps no
 *     pointer after returning and holds no mutable global state, so calls
 *     are re-entrant; the one exception is the static workspace of
 *     fp4kv_decode_attention_noalloc (see there).  Calls on one stream run in
 *     order; calls that write the same cache bytes, or use the same decode
 *     workspace, from different streams race.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default
 *     stream) and the call returns without waiting.  Results are valid once
 *     the stream reaches them.
 *   - Every host-visible argument is checked before any HIP call; a failed
 *     check returns a negative status and touches nothing.  Contents of
 *     device arrays (slots, lengths, page ids) are not visible to the host:
 *     the kernels skip out-of-range entries instead of faulting, as stated
 *     per call.  Inputs must be finite; non-finite K, V or Q give
 *     unspecified results.
 */
#ifndef FP4KV_H
#define FP4KV_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define FP4KV_API __attribute__((visibility("default")))
#else
#define FP4KV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every call returns FP4KV_OK or one of the negative codes. */
enum fp4kv_status {
    FP4KV_OK = 0,
    FP4KV_ERR_INVALID_ARGUMENT = -1,      /* null pointer, negative or inconsistent size */
    FP4KV_ERR_UNSUPPORTED = -2,           /* a valid shape this version does not implement */
    FP4KV_ERR_MISALIGNED = -3,            /* a pointer breaks the stated alignment */
    FP4KV_ERR_WORKSPACE_TOO_SMALL = -4,   /* workspace_bytes below fp4kv_decode_plan's figure */
    FP4KV_ERR_HIP = -5                    /* the HIP runtime reported a launch failure */
};

#define FP4KV_PAGE_SIZE 64                /* tokens per page (the only size in this version) */
#define FP4KV_MAX_GROUP 16                /* query heads per KV head supported */

/* Number formats of a cache.  ("Quantising the KV cache", Concept section,
 * results table: "FP4 E2M1, E4M3 scale per 16" at 4.5 bits per number and
 * "FP8 E4M3, one scale per tensor" at 8; "KV Cache Quantisation", Common
 * questions: FP8 at finer scale granularities, here one fp16 scale per
 * token and KV head, 8 + 16/D bits per number.) */
enum fp4kv_format {
    FP4KV_FORMAT_FP4_E2M1 = 0,            /* E2M1 elements, one E4M3 scale per 16 channels */
    FP4KV_FORMAT_FP8_E4M3 = 1,            /* E4M3 elements, one fp32 scale per tensor (K, V) */
    FP4KV_FORMAT_FP8_E4M3_TOKEN = 2       /* E4M3 elements, one fp16 scale per (token, KV head) */
};

/* Shape of one layer's cache.  ("Quantising the KV cache", Maths section:
 * a token holds 2 x KV heads x head dim numbers per layer; a model keeps one
 * cache per layer, e.g. one buffer per layer or offsets into one buffer.) */
typedef struct fp4kv_cache_params {
    int32_t num_kv_heads;                 /* H_kv >= 1 */
    int32_t head_dim;                     /* D: 64 or 128 */
    int32_t page_size;                    /* tokens per page: FP4KV_PAGE_SIZE */
    int32_t format;                       /* enum fp4kv_format */
    int64_t num_pages;                    /* pages in the pool, >= 1 */
    float k_scale;                        /* FP8: the K tensor's scale, 2^-64 .. 2^64; others: 0 */
    float v_scale;                        /* FP8: the V tensor's scale, 2^-64 .. 2^64; others: 0 */
} fp4kv_cache_params;

/* Byte layout of the cache, filled by fp4kv_cache_layout.  Plain data: it
 * may be copied, stored or sent elsewhere with the cache bytes.
 *
 * The cache is num_pages pages; a page holds one block per KV head; a block
 * (page p, KV head h) starts at p*page_stride + h*head_stride and holds the
 * page's 64 token slots:
 *   K codes   [64 tokens][D/2] bytes       at k_codes_offset: byte i of a
 *             token's row holds channel 2i (low nibble) and 2i+1 (high)
 *   K scales  [64 tokens][D/16]            at k_scales_offset
 *   V codes   [4 slices][D channels][8]    at v_codes_offset: slice j holds
 *             tokens 16j .. 16j+15; byte b of row (j, c) holds channel c of
 *             tokens 16j+2b (low nibble) and 16j+2b+1 (high)
 *   V scales  [4 slices][D/16 blocks][16]  at v_scales_offset: byte t of row
 *             (j, block) is the scale of token 16j+t
 * A nibble is sign << 3 | magnitude code (magnitudes 0, 0.5, 1, 1.5, 2, 3,
 * 4, 6).  A scale byte is an E4M3 code (never 0: a zero scale is stored as
 * the smallest subnormal 2^-9).  Token slot s lives in page s / 64 at
 * offset s % 64.  V is stored channel-major in 16-token slices so that the
 * decode kernels read each channel's tokens contiguously and convert two
 * consecutive tokens of one channel per instruction.
 *
 * FP8 format: a block holds
 *   K codes   [64 tokens][D] bytes         at k_codes_offset (0)
 *   V codes   [4 slices][2 halves][D][8]   at v_codes_offset (64*D): row
 *             (j, h, c) holds channel c of tokens 16j+8h .. 16j+8h+7
 * and no scale planes (k_scales_offset = 64*D and v_scales_offset = 128*D
 * mark empty planes).  A code byte is sign << 7 | E4M3 magnitude code; the
 * stored value is E4M3(code) times the tensor's scale from the params.
 *
 * FP8 format with per-token scales: a block holds
 *   K codes   [64 tokens][D] bytes         at k_codes_offset (0)
 *   K scales  [64 tokens] fp16             at k_scales_offset (64*D)
 *   V codes   as in the FP8 format         at v_codes_offset (64*D + 128)
 *   V scales  [64 tokens] fp16             at v_scales_offset (128*D + 128)
 * The scale of a token's K (or V) row of one KV head is the fp16
 * round-to-nearest-even of amax / 448 over its D channels, saturating at
 * 65504, with 0 replaced by 2^-24; the stored value is E4M3(code) times
 * it. */
typedef struct fp4kv_cache_layout_t {
    fp4kv_cache_params params;
    int64_t block_bytes;                  /* FP4: 64 * D * 9 / 8; FP8: 128 * D; FP8 per token: 128 * D + 256 */
    int64_t k_codes_offset;               /* offsets inside a block */
    int64_t k_scales_offset;
    int64_t v_codes_offset;
    int64_t v_scales_offset;
    int64_t head_stride;                  /* = block_bytes */
    int64_t page_stride;                  /* = num_kv_heads * block_bytes */
    int64_t cache_bytes;                  /* = num_pages * page_stride: exactly 9/16 B (FP8: 1 B; FP8
                                             per token: 1 + 2/D B) per number */
    int64_t bytes_per_token;              /* = 2 * H_kv * D * 9 / 16 (FP8: 2 * H_kv * D; per token:
                                             2 * H_kv * (D + 2)) */
} fp4kv_cache_layout_t;

/* Fill *out from *params.  Host only, no HIP call, pure.
 * Errors: INVALID_ARGUMENT for a null pointer, H_kv < 1, num_pages < 1, an
 * unknown format, FP8 scales not finite and positive or other formats'
 * scales not 0,
 * or a cache size that overflows int64; UNSUPPORTED for head_dim not in
 * {64, 128}, page_size != 64 or FP8 scales outside
 * 2^-64 .. 2^64. */
FP4KV_API int fp4kv_cache_layout(const fp4kv_cache_params *params, fp4kv_cache_layout_t *out);

/* Quantise n_tokens tokens' K and V rows and store them at their slots.
 * ("Quantising the KV cache", Code section: each row is cut into blocks of
 * 16 channels; scale = E4M3 round-to-nearest-even of amax/6, saturating at
 * 448, with 0 replaced by 2^-9; element code = E2M1 round-to-nearest-even of
 * x/scale, saturating at 6, sign kept, also for a zero magnitude.  The
 * quantised K and V are what attention later reads, in place of the real
 * ones.)  A block never spans tokens, so appending never rewrites older
 * tokens and the bytes of a token do not depend on the order of calls or on
 * which tokens share a call (V code bytes shared by two tokens are updated
 * nibble-wise with atomics unless one call covers both).
 * FP8 format ("Quantising the KV cache", Concept section, results table):
 * code = sign << 7 | E4M3 round-to-nearest-even of |x| / scale with the
 * tensor's scale from the layout, saturating at 448, sign kept.  FP8 with
 * per-token scales: the same code under the token's own fp16 scale (see the
 * layout), which is stored beside it.
 *   layout        host, from fp4kv_cache_layout (re-checked).
 *   k, v          device bf16 [n_tokens][H_kv][D], contiguous, 16-B aligned.
 *   n_tokens      >= 0; 0 is a no-op (pointers may then be NULL).
 *   slot_mapping  device int64 [n_tokens], 8-B aligned: slot of token t
 *                 (page * 64 + offset).  Negative slots and slots at or past
 *                 num_pages * 64 are skipped.  Two tokens with one slot race.
 *   cache         device, layout->cache_bytes, 256-B aligned.
 *   stream        hipStream_t or NULL.
 * Errors: INVALID_ARGUMENT (null pointer with n_tokens > 0, n_tokens < 0,
 * layout not produced by fp4kv_cache_layout), MISALIGNED, HIP. */
FP4KV_API int fp4kv_quantize_append(const fp4kv_cache_layout_t *layout,
                          const void *k, const void *v, int64_t n_tokens,
                          const int64_t *slot_mapping, void *cache, void *stream);

/* Split count and workspace bytes for fp4kv_decode_attention.  Host only.
 * The context of every sequence is cut into S chunks of about equal page
 * counts (exact sizes: fp4kv_decode_chunks); one wave attends over each
 * chunk, and workgroups of four waves merge their four chunks into one
 * partial result, so the workspace holds P = ceil(S / 4) partials per
 * (sequence, query head).
 * num_splits > 0 asks for S = num_splits (clamped to max_pages_per_seq and
 * to 4 * 65535, then trimmed so that no chunk starts past page
 * max_pages_per_seq); 0 lets the library choose S, about 16384 chunks in
 * total over batch x H_kv, so that the GPU stays full even when sequence
 * lengths differ, but no more than max_pages_per_seq / 2 (chunks of at
 * least two pages) when that still gives batch x H_kv x S >= 1024.  Each
 * chunk pays a fixed start (its first page's latency, the merge): when every
 * sequence is long and about equally so, chunks of about 32 pages
 * (S = max_pages_per_seq / 32) stream faster than the automatic choice, and
 * for any S a decode call given the shortest length
 * (fp4kv_decode_options.min_seq_len) sizes its chunks for such a batch.
 * *splits_out gets S, *partials_out P and
 * *workspace_bytes_out the workspace fp4kv_decode_attention needs, for the
 * same arguments.
 * Errors: INVALID_ARGUMENT (null pointer, batch < 0, num_q_heads < 1,
 * max_pages_per_seq < 1, num_splits < 0, num_q_heads not a multiple of
 * H_kv), UNSUPPORTED (more than FP4KV_MAX_GROUP query heads per KV head). */
FP4KV_API int fp4kv_decode_plan(const fp4kv_cache_layout_t *layout, int32_t batch, int32_t num_q_heads,
                                int32_t max_pages_per_seq, int32_t num_splits,
                                int32_t *splits_out, int32_t *partials_out, int64_t *workspace_bytes_out);

/* The chunk page counts a decode call with these arguments uses.  Host only;
 * for callers that want to know how the work is cut, and for tests.  With
 * P partials there are 4P chunk slots (chunk 4p + w is wave w of partial
 * p); they tile each sequence's context in order from its first page (with
 * a window: the page of its first query token's window start):
 *   chunk k < *lead_chunks_out  pages [k * LP, (k + 1) * LP)
 *   chunk k >= *lead_chunks_out pages [L + (k - lc) * TP, L + (k - lc + 1) * TP)
 * where lc = *lead_chunks_out, LP = *lead_pages_out, TP = *tail_pages_out and
 * L = lc * LP, each cut at the end of the context.  Usually LP = TP =
 * E = ceil(span / S) (even chunks).  In a grid of at least 1536 workgroups
 * (H_kv x batch x P: twice what 256 CUs hold at once) the last partials take
 * short chunks and the others LP >= E: the workgroups dispatched last are
 * then short ones, so fewer CUs idle while the grid drains.  By default the
 * last floor(P / 2) partials take TP = max(1, 3E / 8) pages.  When
 * min_seq_len (fp4kv_decode_options; 0 here and in the calls without
 * options) says that every sequence covers at least 7/8 of the span
 * (ceil(min_seq_len / 64) >= 7/8 of it), every partial after the lead
 * ones takes TP = max(1, E / 8) pages; the lead partials are the first
 * ceil(768 / (H_kv x batch)) for the FP4 cache (the fewest whose
 * workgroups fill the 768 the GPU holds at once) and, for the FP8 caches,
 * the first max(P - floor(3P / 4), ceil(768 / (H_kv x batch))).  Either cut is used only where it leaves
 * TP < E <= LP.  Arguments as for fp4kv_decode_plan, plus q_tokens >= 1 and
 * window >= 0 as for fp4kv_decode_window_attention (batch x q_tokens x
 * num_q_heads query rows) and min_seq_len >= 0.
 * Errors: as fp4kv_decode_plan, and INVALID_ARGUMENT for a null output,
 * q_tokens < 1, window < 0 or min_seq_len < 0. */
FP4KV_API int fp4kv_decode_chunks(const fp4kv_cache_layout_t *layout, int32_t batch, int32_t q_tokens,
                                  int32_t num_q_heads, int32_t max_pages_per_seq, int32_t window, int32_t num_splits,
                                  int32_t min_seq_len, int32_t *lead_chunks_out, int32_t *lead_pages_out,
                                  int32_t *tail_pages_out);

/* One decode step of attention for `batch` sequences, one query token each,
 * over the packed cache.  ("Quantising the KV cache", Concept and Code
 * sections: every new token reads all cached keys and values; Q is not
 * quantised.  "KV Cache Quantisation", klaylearn, Notes and Common questions:
 * decode reads the cache, so the scales are applied and the codes converted
 * inside the attention kernel, not in a separate pass.)
 * For sequence b and query head h, with G = num_q_heads / H_kv and KV head
 * h / G, over its tokens t < seq_lens[b]:
 *   out[b][h] = sum_t softmax_t(softmax_scale * q[b][h] . K^[t]) * V^[t]
 * where K^, V^ are the stored E2M1 (or E4M3) values times their scales.  The context
 * is cut into splits; each split keeps a running max and sum (online
 * softmax) and a second kernel merges the splits.  Accumulation is fp32.
 *   layout, cache      as above (device cache, 256-B aligned).
 *   q                  device bf16 [batch][num_q_heads][D], 16-B aligned.
 *   batch              >= 0; 0 is a no-op.
 *   seq_lens           device int32 [batch], 4-B aligned; lengths are
 *                      clamped to [0, max_pages_per_seq * 64]; 0 gives a
 *                      zero output row.
 *   page_table         device int32 [batch][max_pages_per_seq]: page id of
 *                      each sequence's i-th 64-token page.  Ids outside
 *                      [0, num_pages) are skipped (their tokens are not
 *                      attended).
 *   softmax_scale      finite and positive (usually 1/sqrt(D)).
 *   num_splits         as for fp4kv_decode_plan.
 *   workspace          device, 256-B aligned, workspace_bytes >= the plan's;
 *                      its contents on entry do not matter.
 *   out                device fp32 [batch][num_q_heads][D], 16-B aligned.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, MISALIGNED, WORKSPACE_TOO_SMALL,
 * HIP.  Equivalent to fp4kv_decode_split followed by fp4kv_decode_combine
 * on the same stream; with one partial per row (at most four chunks) the
 * split kernel writes `out` itself and no combine is launched (the results
 * are the same; fp4kv_decode_with_options can launch the combine anyway). */
FP4KV_API int fp4kv_decode_attention(const fp4kv_cache_layout_t *layout, const void *cache,
                           const void *q, int32_t batch, int32_t num_q_heads,
                           const int32_t *seq_lens, const int32_t *page_table,
                           int32_t max_pages_per_seq, float softmax_scale, int32_t num_splits,
                           void *workspace, int64_t workspace_bytes, float *out, void *stream);

/* The two halves of fp4kv_decode_attention, for callers that time them or
 * merge partial results from several places (for example context chunks
 * attended on different devices, concatenated along the split axis).
 *
 * fp4kv_decode_split takes the arguments of fp4kv_decode_attention except
 * `out` and writes one unnormalised partial result per workgroup to the
 * workspace, laid out as
 *   o   fp32 [batch][P][num_q_heads][D]   at byte 0
 *   ml  fp32 [batch][P][num_q_heads][2]   at byte round_up(batch*P*num_q_heads*D*4, 256)
 * where P is the plan's partial count, m = max_t z_t over the partial's
 * tokens with z_t = log2(e) * softmax_scale * q.k_t, l = sum_t 2^(z_t - m)
 * and o = sum_t 2^(z_t - m) v_t.  A partial without tokens has m = -inf and
 * l = 0, and its o is unspecified (a workgroup whose chunks all lie past the
 * end of its sequence writes only m and l); the combine gives such a partial
 * weight 0 and never uses its o.
 *
 * fp4kv_decode_combine merges P such partials per (sequence, query head):
 *   out = sum_j o_j 2^(m_j - M) / sum_j l_j 2^(m_j - M),  M = max_j m_j,
 * and writes zeros where every partial is empty.  `partials` must be the P
 * of the workspace; workspace_bytes must cover the layout above.
 * Errors: as for fp4kv_decode_attention (combine: INVALID_ARGUMENT for
 * batch < 0, num_q_heads < 1 or partials < 1; UNSUPPORTED for head_dim not
 * in {64, 128}). */
FP4KV_API int fp4kv_decode_split(const fp4kv_cache_layout_t *layout, const void *cache, const void *q,
                       int32_t batch, int32_t num_q_heads, const int32_t *seq_lens,
                       const int32_t *page_table, int32_t max_pages_per_seq, float softmax_scale,
                       int32_t num_splits, void *workspace, int64_t workspace_bytes, void *stream);

FP4KV_API int fp4kv_decode_combine(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t partials,
                                   const void *workspace, int64_t workspace_bytes, float *out, void *stream);

/* fp4kv_decode_attention without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * or harnesses that forbid hipMalloc).  The partial results go to a static
 * device array of FP4KV_NOALLOC_WORKSPACE_BYTES (32 MiB) that the library
 * holds on every GPU it runs on until the process ends; the call itself
 * allocates nothing.  The array's device address is looked up once per
 * device, on the first call with that device current.  Every call on one GPU
 * shares that GPU's array, so calls that overlap on one GPU (different
 * streams, or different threads without ordering) race; calls on one stream
 * run in order.  Nothing in the array has to start at zero: each call
 * overwrites what it reads.
 *   stream       must belong to the current device (or be NULL).
 *   other arguments and results as for fp4kv_decode_attention.
 * Errors: as for fp4kv_decode_attention; WORKSPACE_TOO_SMALL (before any HIP
 * call) when the plan for these arguments needs more than
 * FP4KV_NOALLOC_WORKSPACE_BYTES, i.e. when fp4kv_decode_plan's
 * *workspace_bytes_out exceeds it; HIP if the array's address cannot be
 * looked up. */
#define FP4KV_NOALLOC_WORKSPACE_BYTES (32ll << 20)
FP4KV_API int fp4kv_decode_attention_noalloc(const fp4kv_cache_layout_t *layout, const void *cache,
                                             const void *q, int32_t batch, int32_t num_q_heads,
                                             const int32_t *seq_lens, const int32_t *page_table,
                                             int32_t max_pages_per_seq, float softmax_scale, int32_t num_splits,
                                             float *out, void *stream);

/* One decode step with its own token: for every sequence b with
 * seq_lens[b] >= 1, quantise the new K and V rows k_new[b], v_new[b] (as
 * fp4kv_quantize_append does) into position seq_lens[b] - 1 -- slot
 * page_table[b][(seq_lens[b]-1) / 64] * 64 + (seq_lens[b]-1) % 64 -- then
 * attend over all seq_lens[b] tokens, new one included, exactly as
 * fp4kv_decode_attention.  ("Quantising the KV cache", Code and Concept
 * sections: the hook quantises each new token's K and V, and attention then
 * reads every cached token; "KV Cache Quantisation", Common questions: the
 * gain from a quantised cache depends on fused kernels.)  For the FP4 cache
 * at D = 128 and for the FP8 cache, the decode kernel places the token
 * itself: the one wave that attends over the token's page writes it first,
 * so the step is one kernel plus the combine; otherwise a small kernel places
 * the tokens first.  Results are identical to fp4kv_quantize_append followed
 * by fp4kv_decode_attention.
 *   cache          device, as for the other calls, and written.
 *   k_new, v_new   device bf16 [batch][H_kv][D], 16-B aligned.
 *   other arguments as for fp4kv_decode_attention; seq_lens are the lengths
 *                  including the new token.  A sequence of length 0, or of
 *                  a length above max_pages_per_seq * 64 (whose position is
 *                  not in the table; attention still clamps it), appends
 *                  nothing; an out-of-range page id skips the append (and,
 *                  as always, the page's tokens).  The page that receives a
 *                  sequence's token must not be shared with another
 *                  sequence in the same call.
 * Errors: as for fp4kv_decode_attention, plus INVALID_ARGUMENT for a null
 * k_new or v_new and MISALIGNED.  fp4kv_decode_append_split is the same
 * without the combine (see fp4kv_decode_split). */
FP4KV_API int fp4kv_decode_append_attention(const fp4kv_cache_layout_t *layout, void *cache,
                                            const void *k_new, const void *v_new, const void *q,
                                            int32_t batch, int32_t num_q_heads, const int32_t *seq_lens,
                                            const int32_t *page_table, int32_t max_pages_per_seq,
                                            float softmax_scale, int32_t num_splits, void *workspace,
                                            int64_t workspace_bytes, float *out, void *stream);

FP4KV_API int fp4kv_decode_append_split(const fp4kv_cache_layout_t *layout, void *cache, const void *k_new,
                                        const void *v_new, const void *q, int32_t batch, int32_t num_q_heads,
                                        const int32_t *seq_lens, const int32_t *page_table,
                                        int32_t max_pages_per_seq, float softmax_scale, int32_t num_splits,
                                        void *workspace, int64_t workspace_bytes, void *stream);

/* Attention of several consecutive query tokens per sequence over the
 * packed cache, with causal masking: q_tokens query tokens sit at the last
 * q_tokens positions of each context (speculative tokens being verified, or
 * a chunk of a prefill), and query token i of sequence b attends over its
 * first seq_lens[b] - (q_tokens - 1 - i) tokens.  Their K and V must already
 * be in the cache (fp4kv_quantize_append).  ("Quantising the KV cache",
 * Concept: attention reads every cached token up to the query's own; the
 * same codec and kernels as fp4kv_decode_attention.)  The matrix-core
 * kernels take q_tokens x (num_q_heads / H_kv) <= 16 query columns per KV
 * head, so one pass over the cache serves all of them.
 *   q     device bf16 [batch][q_tokens][num_q_heads][D], 16-B aligned.
 *   out   device fp32 [batch][q_tokens][num_q_heads][D], 16-B aligned.
 *   workspace  as fp4kv_decode_plan gives for q_tokens * num_q_heads query
 *         heads (its group limit is the 16 columns above).
 *   other arguments as for fp4kv_decode_attention.  A query token whose
 *   limit is 0 or below gets a zero row.  q_tokens = 1 is
 *   fp4kv_decode_attention.
 * Errors: as for fp4kv_decode_attention; INVALID_ARGUMENT for q_tokens < 1;
 * UNSUPPORTED for more than 16 query columns per KV head. */
FP4KV_API int fp4kv_decode_multi_attention(const fp4kv_cache_layout_t *layout, const void *cache,
                                           const void *q, int32_t batch, int32_t q_tokens, int32_t num_q_heads,
                                           const int32_t *seq_lens, const int32_t *page_table,
                                           int32_t max_pages_per_seq, float softmax_scale, int32_t num_splits,
                                           void *workspace, int64_t workspace_bytes, float *out, void *stream);

/* Sliding-window attention over the packed cache: as
 * fp4kv_decode_multi_attention (q_tokens query tokens per sequence at the
 * end of each context, causal), and query token i sees only the last
 * `window` tokens of its prefix, positions max(0, L_i - window) .. L_i - 1
 * with L_i = seq_lens[b] - (q_tokens - 1 - i); window = 0 means no window.
 * Only the pages that hold those tokens are read.  ("Week 6 -- FP4 KV Caches
 * and Bounded Replay", Overview and Core Concepts: sliding-window layers keep
 * their KV in FP8 and attend over the last n_win tokens; the same cache
 * formats and kernels as fp4kv_decode_attention.)
 * fp4kv_decode_window_plan gives the split count S, partials P and the
 * workspace bytes for the same arguments (the splits cover the window's
 * pages, not the whole table).
 *   window       >= 0.
 *   other arguments as for fp4kv_decode_multi_attention.
 * Errors: as for fp4kv_decode_multi_attention; INVALID_ARGUMENT for a
 * negative window. */
FP4KV_API int fp4kv_decode_window_plan(const fp4kv_cache_layout_t *layout, int32_t batch, int32_t q_tokens,
                                       int32_t num_q_heads, int32_t max_pages_per_seq, int32_t window,
                                       int32_t num_splits, int32_t *splits_out, int32_t *partials_out,
                                       int64_t *workspace_bytes_out);

FP4KV_API int fp4kv_decode_window_attention(const fp4kv_cache_layout_t *layout, const void *cache,
                                            const void *q, int32_t batch, int32_t q_tokens,
                                            int32_t num_q_heads, const int32_t *seq_lens,
                                            const int32_t *page_table, int32_t max_pages_per_seq,
                                            int32_t window, float softmax_scale, int32_t num_splits,
                                            void *workspace, int64_t workspace_bytes, float *out, void *stream);

/* Choices inside a decode call, and what the caller knows of the batch;
 * the other entry points use FP4KV_DECODE_KERNEL_AUTO,
 * FP4KV_DECODE_MERGE_AUTO and min_seq_len 0.  Every choice gives the same
 * results within the attention tolerance, and the same split kernel over
 * the same chunks gives the same bits whatever the merge. */
enum fp4kv_decode_kernel {
    FP4KV_DECODE_KERNEL_AUTO = 0,         /* FP8 cache: its kernel; FP4: MFMA_STAGED at D = 128, else MFMA_DIRECT */
    FP4KV_DECODE_KERNEL_MFMA_STAGED = 1,  /* FP4, D = 128: matrix cores, pages staged through LDS */
    FP4KV_DECODE_KERNEL_MFMA_DIRECT = 2,  /* FP4: matrix cores, operands loaded straight into registers */
    FP4KV_DECODE_KERNEL_VALU = 3          /* FP4, one query token, no window: vector ALU only */
};
enum fp4kv_decode_merge {
    FP4KV_DECODE_MERGE_AUTO = 0,          /* one partial per row: the split kernel writes out; else a combine */
    FP4KV_DECODE_MERGE_COMBINE_KERNEL = 1, /* always a separate combine kernel */
    FP4KV_DECODE_MERGE_NONE = 2           /* the split kernel alone: partials left in the workspace as
                                             fp4kv_decode_split leaves them; `out` is not used (may be NULL) */
};
typedef struct fp4kv_decode_options {
    int32_t kernel;                       /* enum fp4kv_decode_kernel */
    int32_t merge;                        /* enum fp4kv_decode_merge */
    int32_t min_seq_len;                  /* host knowledge: every seq_lens[b] is at least this (0: nothing
                                             known; negative: INVALID_ARGUMENT).  It only decides how the
                                             context is cut into chunks (fp4kv_decode_chunks): when every
                                             sequence covers at least 7/8 of the span, the last chunks are
                                             made shorter than for a ragged batch.  Every cut covers the same
                                             tokens, so a wrong value costs time, never correctness (results
                                             differ from the unhinted call's by rounding only). */
} fp4kv_decode_options;

/* Every decode entry point in one call, with explicit choices: append the
 * step's token when k_new and v_new are given (both or neither; then
 * q_tokens must be 1 and window 0), q_tokens query tokens per sequence,
 * sliding window `window` (0: none), as fp4kv_decode_append_attention,
 * fp4kv_decode_multi_attention and fp4kv_decode_window_attention describe.
 * `options` (host; NULL: AUTO, AUTO, 0) chooses the split kernel, whether a
 * separate combine kernel merges the partials (or none: the split kernel
 * alone, as fp4kv_decode_split; then `out` may be NULL) and gives the
 * shortest length's lower bound that sizes the chunks.  The workspace is
 * sized by fp4kv_decode_window_plan for the same arguments
 * (fp4kv_decode_plan when q_tokens = 1 and window = 0).
 * Errors: as for those calls; INVALID_ARGUMENT for an unknown option value,
 * a negative min_seq_len or only one of k_new, v_new; UNSUPPORTED for a kernel that does not serve
 * the cache format, head size, query tokens or window, or an append with
 * q_tokens > 1 or a window. */
FP4KV_API int fp4kv_decode_with_options(const fp4kv_cache_layout_t *layout, void *cache, const void *k_new,
                                        const void *v_new, const void *q, int32_t batch, int32_t q_tokens,
                                        int32_t num_q_heads, const int32_t *seq_lens, const int32_t *page_table,
                                        int32_t max_pages_per_seq, int32_t window, float softmax_scale,
                                        int32_t num_splits, void *workspace, int64_t workspace_bytes, float *out,
                                        const fp4kv_decode_options *options, void *stream);

/* Measurement utility, not a step of the method: reads `bytes` of device
 * memory at `buf` (device) once with 16-byte loads and discards the data.
 * Each wave reads whole 9216-byte blocks, the size of one page of one KV head
 * at D = 128, so the rate it reaches is the achievable HBM read rate for the
 * decode kernel's access pattern.  `bytes` must be a positive multiple of
 * 9216 and `buf` 256-byte aligned; `sink` (device, 4 bytes) is written only
 * if the XOR of everything read equals 0x9E3779B9, which keeps the loads
 * from being optimised away.  Returns FP4KV_OK, or INVALID_ARGUMENT /
 * MISALIGNED before any HIP call, or FP4KV_ERR_HIP. */
FP4KV_API int fp4kv_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/* Measurement utility, not a step of the method: the same one-pass read of
 * `bytes` at `buf` with a chosen shape, to find the achievable read rate.
 * Each wave reads whole stretches of 64 * 16 * loads_per_lane bytes (16-byte
 * non-temporal loads, loads_per_lane of them per lane in flight together)
 * in a grid-stride loop over `workgroups` workgroups of four waves, into
 * registers (to_lds = 0) or straight into LDS (to_lds = 1, as the decode
 * kernels copy pages).  loads_per_lane is 1, 2, 4, 8 or 16; `bytes` a
 * positive multiple of 1024 * loads_per_lane; `buf` 1024-byte aligned; `sink`
 * as for fp4kv_read_probe.  Returns FP4KV_OK, or INVALID_ARGUMENT /
 * MISALIGNED before any HIP call, or FP4KV_ERR_HIP. */
FP4KV_API int fp4kv_read_probe_config(const void *buf, int64_t bytes, int32_t loads_per_lane, int32_t workgroups,
                                      int32_t to_lds, uint32_t *sink, void *stream);

/* Measurement utility, not a step of the method: the achievable rate of a
 * kernel that streams reads and writes in a given proportion.  `units`
 * waves' worth of work, in a grid-stride loop over `workgroups` workgroups of
 * four waves: unit u reads read_bytes contiguous bytes at src + u *
 * read_bytes (128 bytes per lane in flight) and then writes write_bytes
 * contiguous bytes at dst + u * write_bytes.  paired = 0: each load
 * instruction reads a whole kilobyte (16 bytes per lane); paired = 1: lane l
 * reads bytes [32 l, 32 l + 32) of each 2 KB row in two 16-byte loads, the
 * pattern of the quantiser, which holds a 16-channel bf16 block per lane.
 * read_bytes a positive multiple of 8192, write_bytes a multiple of 1024
 * (0: no writes, dst may be NULL); src and dst 1024-byte aligned and at
 * least units * read_bytes and units * write_bytes long (not checkable:
 * the caller's obligation); sink as for fp4kv_read_probe.  Returns
 * FP4KV_OK, or INVALID_ARGUMENT / MISALIGNED before any HIP call, or
 * FP4KV_ERR_HIP. */
FP4KV_API int fp4kv_stream_probe(const void *src, void *dst, int64_t units, int32_t read_bytes, int32_t write_bytes,
                                 int32_t paired, int32_t workgroups, uint32_t *sink, void *stream);

/* Static text for a status code (never NULL). */
FP4KV_API const char *fp4kv_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch.  0.2.0 added
 * min_seq_len to fp4kv_decode_options (and to fp4kv_decode_chunks' arguments)
 * and FP4KV_DECODE_MERGE_NONE; a caller built against another version's
 * header must not call this library. */
#define FP4KV_VERSION 200
FP4KV_API int fp4kv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4KV_H */
