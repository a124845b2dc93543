// Host side of the FP4 KV-cache C ABI: layout arithmetic, argument checks,
// split planning and kernel launches.  Every check runs before the first HIP
// call, so a rejected call has no effect on the device.
#include "fp4kv.h"

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <limits>

#include <hip/hip_runtime.h>

#include "fp4kv_internal.h"

namespace {

constexpr int32_t kPage = FP4KV_PAGE_SIZE;
constexpr int32_t kTargetWaves = 16384;   // context chunks (one wave each): 4x the waves 256 CUs hold at once, so ragged lengths balance
constexpr int64_t kMinAutoChunkPages = 2;  // automatic plans: pages per chunk at least ...
constexpr int64_t kMinAutoChunks = 1024;   // ... unless that leaves fewer chunks than this
constexpr int32_t kChunksPerGroup = 4;   // chunks merged inside one workgroup
constexpr int64_t kMaxPartials = 65535;  // partials per row: the split kernel's third grid dimension
constexpr int64_t kResidentGroups = 768;  // split-kernel workgroups resident at once: 256 CUs x 3

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// FP8 per-tensor scales the quantiser handles exactly: 2^-64 .. 2^64.
bool in_scale_range(float s) { return s >= 0x1p-64f && s <= 0x1p64f; }

// Layout of one (page, KV head) block.  FP4: K codes, K scales, V codes, V
// scales.  FP8: K codes, V codes (empty scale planes at their ends).
int fill_layout(const fp4kv_cache_params &p, fp4kv_cache_layout_t *out)
{
    if (p.num_kv_heads < 1 || p.num_pages < 1)
        return FP4KV_ERR_INVALID_ARGUMENT;
    const bool fp8 = p.format == FP4KV_FORMAT_FP8_E4M3;
    const bool fp8_token = p.format == FP4KV_FORMAT_FP8_E4M3_TOKEN;
    if (p.format != FP4KV_FORMAT_FP4_E2M1 && !fp8 && !fp8_token)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (fp8 ? !(std::isfinite(p.k_scale) && p.k_scale > 0.0f && std::isfinite(p.v_scale) && p.v_scale > 0.0f)
            : (p.k_scale != 0.0f || p.v_scale != 0.0f))
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (fp8 && !(in_scale_range(p.k_scale) && in_scale_range(p.v_scale)))
        return FP4KV_ERR_UNSUPPORTED;
    if (p.head_dim != 64 && p.head_dim != 128)
        return FP4KV_ERR_UNSUPPORTED;
    if (p.page_size != kPage)
        return FP4KV_ERR_UNSUPPORTED;
    const int64_t D = p.head_dim;
    const int64_t codes = fp8 || fp8_token ? kPage * D : kPage * D / 2;
    const int64_t scales = fp8 ? 0 : fp8_token ? kPage * 2 : kPage * D / 16;
    const int64_t block = 2 * (codes + scales);   // FP4: 64 * D * 9 / 8; FP8: 128 * D; per token: 128 * D + 256
    const int64_t page_stride = block * p.num_kv_heads;
    if (p.num_pages > std::numeric_limits<int64_t>::max() / page_stride)
        return FP4KV_ERR_INVALID_ARGUMENT;
    fp4kv_cache_layout_t L{};
    L.params = p;
    L.block_bytes = block;
    L.k_codes_offset = 0;
    L.k_scales_offset = codes;
    L.v_codes_offset = codes + scales;
    L.v_scales_offset = 2 * codes + scales;
    L.head_stride = block;
    L.page_stride = page_stride;
    L.cache_bytes = page_stride * p.num_pages;
    L.bytes_per_token = page_stride / kPage;
    *out = L;
    return FP4KV_OK;
}

// A layout passed back in must be exactly what fp4kv_cache_layout produces.
int check_layout(const fp4kv_cache_layout_t *L)
{
    if (!L)
        return FP4KV_ERR_INVALID_ARGUMENT;
    fp4kv_cache_layout_t ref;
    const int rc = fill_layout(L->params, &ref);
    if (rc != FP4KV_OK)
        return rc;
    if (ref.block_bytes != L->block_bytes || ref.k_codes_offset != L->k_codes_offset ||
        ref.k_scales_offset != L->k_scales_offset || ref.v_codes_offset != L->v_codes_offset ||
        ref.v_scales_offset != L->v_scales_offset || ref.head_stride != L->head_stride ||
        ref.page_stride != L->page_stride || ref.cache_bytes != L->cache_bytes ||
        ref.bytes_per_token != L->bytes_per_token)
        return FP4KV_ERR_INVALID_ARGUMENT;
    return FP4KV_OK;
}

fp4kv::CacheGeom geom_of(const fp4kv_cache_layout_t &L)
{
    fp4kv::CacheGeom g;
    g.num_kv_heads = L.params.num_kv_heads;
    g.head_dim = L.params.head_dim;
    g.num_pages = L.params.num_pages;
    g.k_codes_off = L.k_codes_offset;
    g.k_scales_off = L.k_scales_offset;
    g.v_codes_off = L.v_codes_offset;
    g.v_scales_off = L.v_scales_offset;
    g.head_stride = L.head_stride;
    g.page_stride = L.page_stride;
    g.token_scales = L.params.format == FP4KV_FORMAT_FP8_E4M3_TOKEN;
    g.fp8 = L.params.format == FP4KV_FORMAT_FP8_E4M3 || g.token_scales;
    g.k_scale = L.params.k_scale;
    g.v_scale = L.params.v_scale;
    return g;
}

struct Plan {
    int32_t splits;
    int32_t pages_per_split;
    int32_t partials;          // ceil(splits / kChunksPerGroup)
    int64_t ws_o_bytes;        // fp32 partial outputs
    int64_t ws_bytes;          // total, including the (max, sum) pairs
};

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int make_plan(const fp4kv_cache_layout_t &L, int32_t batch, int32_t num_q_heads,
              int32_t max_pages, int32_t requested, Plan *plan)
{
    if (batch < 0 || num_q_heads < 1 || max_pages < 1 || requested < 0)
        return FP4KV_ERR_INVALID_ARGUMENT;
    const int32_t hkv = L.params.num_kv_heads;
    if (num_q_heads % hkv != 0)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (num_q_heads / hkv > FP4KV_MAX_GROUP)
        return FP4KV_ERR_UNSUPPORTED;
    int64_t s = requested;
    if (s == 0) {
        const int64_t units = static_cast<int64_t>(batch > 0 ? batch : 1) * hkv;
        s = (kTargetWaves + units - 1) / units;
        // chunks of one page are mostly fixed cost: at least two pages each,
        // as long as that still leaves enough chunks to spread over the GPU
        // (a tiny batch is faster with one page per wave, in parallel)
        const int64_t most = max_pages / kMinAutoChunkPages;
        if (most > 0 && units * most >= kMinAutoChunks)
            s = s > most ? most : s;
    }
    if (s > max_pages)
        s = max_pages;
    if (s > static_cast<int64_t>(kChunksPerGroup) * kMaxPartials)
        s = static_cast<int64_t>(kChunksPerGroup) * kMaxPartials;
    if (s < 1)
        s = 1;
    const int64_t pps = (max_pages + s - 1) / s;
    s = (max_pages + pps - 1) / pps;                          // no split starts past the last page
    plan->splits = static_cast<int32_t>(s);
    plan->pages_per_split = static_cast<int32_t>(pps);
    plan->partials = static_cast<int32_t>((s + kChunksPerGroup - 1) / kChunksPerGroup);
    const int64_t rows = static_cast<int64_t>(batch) * num_q_heads * plan->partials;
    plan->ws_o_bytes = round_up(rows * L.params.head_dim * 4, 256);
    plan->ws_bytes = plan->ws_o_bytes + round_up(rows * 2 * 4, 256);
    return FP4KV_OK;
}

// Chunk page counts of a plan (chunk_first_page in the kernels): the first
// lead_chunks chunks hold lead_pages pages, the rest tail_pages.  Even
// chunks of pages_per_split, except in a grid of at least twice the
// workgroups the GPU runs at once: there the workgroups the grid starts last
// are given short chunks (longest first), so that few slots idle while it
// drains, and the earlier partials share out the remaining pages.  How far
// that can go depends on the lengths, which only the caller knows:
//   - by default the last half of the partials take chunks of 3/8 of the
//     even size;
//   - when the caller promises that every sequence covers at least 7/8 of
//     the span (min_span: pages each sequence is known to cover, 0 when
//     nothing is known), every partial after the lead ones takes chunks of
//     1/8 of the even size (at least one page).  The lead partials are, for
//     the FP4 cache, the fewest whose workgroups fill the GPU's resident
//     slots at least once; for the FP8 caches a quarter of the partials, or
//     that many if a quarter does not fill the slots.
// (Measured on the 32 x 32K batch at 64 chunks and the paged 64-sequence
// batch: the second cut gains about 6 % on the first -- with FP4 pages,
// lead partials beyond one generation's worth are 1.6 % slower, fewer than
// one generation's worth (64 sequences, one partial of 512) 7 % slower, with the
// FP8 caches' 16 KB pages fewer than a quarter are 1-4 % slower -- but on
// the second it packs a short sequence's pages into one long lead chunk
// whose workgroup's other waves idle, and it holds the long sequences in
// few long workgroups.)
struct ChunkSizes {
    int32_t lead_chunks, lead_pages, tail_pages;
};

ChunkSizes chunk_sizes(const fp4kv_cache_layout_t &L, int32_t batch, const Plan &plan, int64_t span,
                       int64_t min_span)
{
    const int64_t chunks = static_cast<int64_t>(plan.partials) * kChunksPerGroup;
    ChunkSizes cs{static_cast<int32_t>(chunks), plan.pages_per_split, plan.pages_per_split};
    const int64_t units = static_cast<int64_t>(L.params.num_kv_heads) * batch;     // workgroups per partial
    const int64_t groups = units * plan.partials;
    const bool uniform = min_span > 0 && 8 * min_span >= 7 * span;
    const bool fp4 = L.params.format == FP4KV_FORMAT_FP4_E2M1;
    const int64_t fill = (kResidentGroups + units - 1) / std::max<int64_t>(1, units);   // lead partials to fill the GPU
    const int64_t lead_parts = !uniform ? plan.partials - plan.partials / 2
                               : fp4    ? fill
                                        : std::max<int64_t>(fill, plan.partials - plan.partials * 3 / 4);
    const int64_t tail_parts = plan.partials - lead_parts;
    if (groups < 2 * kResidentGroups || tail_parts < 1)
        return cs;
    const int64_t tail = std::max<int64_t>(1, plan.pages_per_split * (uniform ? 1 : 3) / 8);
    const int64_t lead_chunks = lead_parts * kChunksPerGroup;
    const int64_t lead = (span - tail_parts * kChunksPerGroup * tail + lead_chunks - 1) / lead_chunks;
    if (tail < plan.pages_per_split && lead >= plan.pages_per_split) {
        cs.lead_chunks = static_cast<int32_t>(lead_chunks);
        cs.lead_pages = static_cast<int32_t>(lead);
        cs.tail_pages = static_cast<int32_t>(tail);
    }
    return cs;
}

// Pages of the span every sequence covers when each is at least min_seq_len
// tokens long (0: nothing known).
int64_t promised_span(int64_t span, int32_t min_seq_len)
{
    const int64_t pages = (static_cast<int64_t>(min_seq_len) + kPage - 1) / kPage;
    return pages < span ? pages : span;
}

}  // namespace

extern "C" {

int fp4kv_cache_layout(const fp4kv_cache_params *params, fp4kv_cache_layout_t *out)
{
    if (!params || !out)
        return FP4KV_ERR_INVALID_ARGUMENT;
    return fill_layout(*params, out);
}

int fp4kv_quantize_append(const fp4kv_cache_layout_t *layout, const void *k, const void *v,
                          int64_t n_tokens, const int64_t *slot_mapping, void *cache, void *stream)
{
    int rc = check_layout(layout);
    if (rc != FP4KV_OK)
        return rc;
    if (n_tokens < 0)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (n_tokens == 0)
        return FP4KV_OK;
    if (!k || !v || !slot_mapping || !cache)
        return FP4KV_ERR_INVALID_ARGUMENT;
    const int64_t per_token = static_cast<int64_t>(layout->params.num_kv_heads) * (layout->params.head_dim / 16);
    if (n_tokens > static_cast<int64_t>(std::numeric_limits<int32_t>::max()) * 256 / per_token)
        return FP4KV_ERR_UNSUPPORTED;                        // the launch grid would not fit
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8) || !aligned(cache, 256))
        return FP4KV_ERR_MISALIGNED;
    const hipError_t e = fp4kv::launch_quantize_append(
        geom_of(*layout), static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
        n_tokens, slot_mapping, static_cast<uint8_t *>(cache), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP;
}

int fp4kv_decode_plan(const fp4kv_cache_layout_t *layout, int32_t batch, int32_t num_q_heads,
                      int32_t max_pages_per_seq, int32_t num_splits, int32_t *splits_out,
                      int32_t *partials_out, int64_t *workspace_bytes_out)
{
    int rc = check_layout(layout);
    if (rc != FP4KV_OK)
        return rc;
    if (!splits_out || !partials_out || !workspace_bytes_out)
        return FP4KV_ERR_INVALID_ARGUMENT;
    Plan plan;
    rc = make_plan(*layout, batch, num_q_heads, max_pages_per_seq, num_splits, &plan);
    if (rc != FP4KV_OK)
        return rc;
    *splits_out = plan.splits;
    *partials_out = plan.partials;
    *workspace_bytes_out = plan.ws_bytes;
    return FP4KV_OK;
}

}  // extern "C"

namespace {

int32_t window_span_pages(int32_t max_pages, int32_t q_tokens, int32_t window);

}  // namespace

extern "C" {

int fp4kv_decode_chunks(const fp4kv_cache_layout_t *layout, int32_t batch, int32_t q_tokens, int32_t num_q_heads,
                        int32_t max_pages_per_seq, int32_t window, int32_t num_splits, int32_t min_seq_len,
                        int32_t *lead_chunks_out, int32_t *lead_pages_out, int32_t *tail_pages_out)
{
    int rc = check_layout(layout);
    if (rc != FP4KV_OK)
        return rc;
    if (!lead_chunks_out || !lead_pages_out || !tail_pages_out || q_tokens < 1 || window < 0 || num_q_heads < 1 ||
        min_seq_len < 0 || static_cast<int64_t>(q_tokens) * num_q_heads > std::numeric_limits<int32_t>::max())
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (max_pages_per_seq < 1)
        return FP4KV_ERR_INVALID_ARGUMENT;
    const int32_t span = window_span_pages(max_pages_per_seq, q_tokens, window);
    Plan plan;
    rc = make_plan(*layout, batch, q_tokens * num_q_heads, span, num_splits, &plan);
    if (rc != FP4KV_OK)
        return rc;
    const ChunkSizes cs = chunk_sizes(*layout, batch, plan, span, promised_span(span, min_seq_len));
    *lead_chunks_out = cs.lead_chunks;
    *lead_pages_out = cs.lead_pages;
    *tail_pages_out = cs.tail_pages;
    return FP4KV_OK;
}

}  // extern "C"

namespace {

// Checks shared by fp4kv_decode_split and fp4kv_decode_attention; fills the
// kernel arguments (out is left null).
// Pages a split plan has to cover: the whole table, or with a sliding
// window the pages from the first query token's window start to the end of
// the context (at most ceil((window + q_tokens - 1) / 64) + 1).
int32_t window_span_pages(int32_t max_pages, int32_t q_tokens, int32_t window)
{
    if (window <= 0)
        return max_pages;
    const int64_t span = (static_cast<int64_t>(window) + q_tokens - 1 + kPage - 1) / kPage + 1;
    return static_cast<int32_t>(span < max_pages ? span : max_pages);
}

int prepare_split(const fp4kv_cache_layout_t *layout, const void *cache, const void *q,
                  int32_t batch, int32_t num_q_heads, const int32_t *seq_lens,
                  const int32_t *page_table, int32_t max_pages_per_seq, float softmax_scale,
                  int32_t num_splits, void *workspace, int64_t workspace_bytes,
                  fp4kv::DecodeArgs *a, int32_t q_tokens = 1, int32_t window = 0, int32_t min_seq_len = 0)
{
    int rc = check_layout(layout);
    if (rc != FP4KV_OK)
        return rc;
    if (window < 0 || min_seq_len < 0)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (q_tokens < 1 || num_q_heads < 1 || num_q_heads % layout->params.num_kv_heads ||
        static_cast<int64_t>(q_tokens) * num_q_heads > std::numeric_limits<int32_t>::max())
        return FP4KV_ERR_INVALID_ARGUMENT;
    Plan plan;
    // several query tokens: the plan's rows (and its group limit) count
    // q_tokens x num_q_heads query rows
    rc = make_plan(*layout, batch, q_tokens * num_q_heads, window_span_pages(max_pages_per_seq, q_tokens, window),
                   num_splits, &plan);
    if (rc != FP4KV_OK)
        return rc;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f))
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (static_cast<int64_t>(max_pages_per_seq) * kPage > std::numeric_limits<int32_t>::max())
        return FP4KV_ERR_UNSUPPORTED;
    if (batch > 65535 || layout->params.num_kv_heads > 65535)
        return FP4KV_ERR_UNSUPPORTED;                        // grid y/z limits
    if (batch == 0)
        return FP4KV_OK;
    if (!cache || !q || !seq_lens || !page_table || !workspace)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (!aligned(cache, 256) || !aligned(q, 16) || !aligned(seq_lens, 4) ||
        !aligned(page_table, 4) || !aligned(workspace, 256))
        return FP4KV_ERR_MISALIGNED;
    if (workspace_bytes < plan.ws_bytes)
        return FP4KV_ERR_WORKSPACE_TOO_SMALL;

    a->geom = geom_of(*layout);
    a->cache = static_cast<const uint8_t *>(cache);
    a->q = static_cast<const uint16_t *>(q);
    a->seq_lens = seq_lens;
    a->page_table = page_table;
    a->batch = batch;
    a->num_q_heads = num_q_heads;
    a->group = num_q_heads / layout->params.num_kv_heads;
    a->q_tokens = q_tokens;
    a->window = window;
    a->max_pages = max_pages_per_seq;
    a->splits = plan.splits;
    a->pages_per_split = plan.pages_per_split;
    a->partials = plan.partials;
    const int32_t span = window_span_pages(max_pages_per_seq, q_tokens, window);
    const ChunkSizes cs = chunk_sizes(*layout, batch, plan, span, promised_span(span, min_seq_len));
    a->lead_chunks = cs.lead_chunks;
    a->lead_pages = cs.lead_pages;
    a->tail_pages = cs.tail_pages;
    a->staged = true;
    // scores are kept in base 2; an FP8 cache's K tensor scale multiplies every score
    const double k_scale = layout->params.format == FP4KV_FORMAT_FP8_E4M3 ? layout->params.k_scale : 1.0;
    a->scale_log2e = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634 * k_scale);
    a->ws_o = static_cast<float *>(workspace);
    a->ws_ml = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + plan.ws_o_bytes);

    a->out = nullptr;
    a->k_new = a->v_new = nullptr;
    a->cache_w = nullptr;
    return FP4KV_OK;
}

// The step's own token for the append variants: rows [batch][H_kv][D].
int prepare_append(void *cache, const void *k_new, const void *v_new, fp4kv::DecodeArgs *a)
{
    if (!k_new || !v_new)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (!aligned(k_new, 16) || !aligned(v_new, 16))
        return FP4KV_ERR_MISALIGNED;
    a->k_new = static_cast<const uint16_t *>(k_new);
    a->v_new = static_cast<const uint16_t *>(v_new);
    a->cache_w = static_cast<uint8_t *>(cache);
    return FP4KV_OK;
}

int64_t partial_o_bytes(int32_t batch, int32_t num_q_heads, int32_t partials, int32_t head_dim)
{
    return round_up(static_cast<int64_t>(batch) * num_q_heads * partials * head_dim * 4, 256);
}

// The split kernel a call asks for (FP4KV_DECODE_KERNEL_AUTO: the default
// for the cache), if it serves these arguments.
int choose_kernel(const fp4kv::DecodeArgs &a, int32_t requested, fp4kv::SplitKernel *out)
{
    using fp4kv::SplitKernel;
    const bool fp8 = a.geom.fp8;
    switch (requested) {
    case FP4KV_DECODE_KERNEL_AUTO:
        *out = fp8 ? SplitKernel::fp8 : a.geom.head_dim == 128 ? SplitKernel::mfma_staged : SplitKernel::mfma_direct;
        return FP4KV_OK;
    case FP4KV_DECODE_KERNEL_MFMA_STAGED:
        if (fp8 || a.geom.head_dim != 128)
            return FP4KV_ERR_UNSUPPORTED;
        *out = SplitKernel::mfma_staged;
        return FP4KV_OK;
    case FP4KV_DECODE_KERNEL_MFMA_DIRECT:
        if (fp8)
            return FP4KV_ERR_UNSUPPORTED;
        *out = SplitKernel::mfma_direct;
        return FP4KV_OK;
    case FP4KV_DECODE_KERNEL_VALU:
        if (fp8 || a.q_tokens > 1 || a.window > 0)
            return FP4KV_ERR_UNSUPPORTED;
        *out = SplitKernel::valu;
        return FP4KV_OK;
    default:
        return FP4KV_ERR_INVALID_ARGUMENT;
    }
}

// How a call ends, fixed by its checks before any launch.
struct Finish {
    fp4kv::SplitKernel kernel;
    bool combine;                // a combine kernel after the split kernel (else the split kernel writes out)
    bool partials_only;          // the split kernel alone, partials left in the workspace
};


// Checks of `out` and of the options (null: defaults) for a call whose
// split arguments are in `a`.
int check_finish(const fp4kv::DecodeArgs &a, const float *out, const fp4kv_decode_options *opts, Finish *f)
{
    const int32_t kernel = opts ? opts->kernel : FP4KV_DECODE_KERNEL_AUTO;
    const int32_t merge = opts ? opts->merge : FP4KV_DECODE_MERGE_AUTO;
    if (merge != FP4KV_DECODE_MERGE_AUTO && merge != FP4KV_DECODE_MERGE_COMBINE_KERNEL &&
        merge != FP4KV_DECODE_MERGE_NONE)
        return FP4KV_ERR_INVALID_ARGUMENT;
    f->partials_only = merge == FP4KV_DECODE_MERGE_NONE;
    if (!f->partials_only) {
        if (!out)
            return FP4KV_ERR_INVALID_ARGUMENT;
        if (!aligned(out, 16))
            return FP4KV_ERR_MISALIGNED;
    }
    const int rc = choose_kernel(a, kernel, &f->kernel);
    if (rc != FP4KV_OK)
        return rc;
    // With one partial per row the split kernel writes the final rows itself
    // (the combine's weight would be exactly 1) and no combine is launched.
    f->combine = !f->partials_only && (a.partials != 1 || merge == FP4KV_DECODE_MERGE_COMBINE_KERNEL);
    return FP4KV_OK;
}

// The launches of a checked call.
int run_decode(fp4kv::DecodeArgs &a, const Finish &f, float *out, hipStream_t st)
{
    a.out = f.combine || f.partials_only ? nullptr : out;
    hipError_t e = fp4kv::launch_decode_split(a, f.kernel, st);
    if (e != hipSuccess)
        return FP4KV_ERR_HIP;
    if (!f.combine)
        return FP4KV_OK;
    e = fp4kv::launch_decode_combine(a.ws_o, a.ws_ml, a.batch, a.q_tokens * a.num_q_heads, a.partials,
                                     a.geom.head_dim, out, st);
    return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP;
}

// Every attention entry point: split arguments, the optional appended token,
// then the finish.
int decode_call(const fp4kv_cache_layout_t *layout, void *cache, const void *k_new, const void *v_new, bool append,
                const void *q, int32_t batch, int32_t q_tokens, int32_t num_q_heads, const int32_t *seq_lens,
                const int32_t *page_table, int32_t max_pages_per_seq, int32_t window, float softmax_scale,
                int32_t num_splits, void *workspace, int64_t workspace_bytes, float *out,
                const fp4kv_decode_options *opts, void *stream)
{
    fp4kv::DecodeArgs a;
    int rc = prepare_split(layout, cache, q, batch, num_q_heads, seq_lens, page_table, max_pages_per_seq,
                           softmax_scale, num_splits, workspace, workspace_bytes, &a, q_tokens, window,
                           opts ? opts->min_seq_len : 0);
    if (rc != FP4KV_OK || batch == 0)
        return rc;
    if (append) {
        rc = prepare_append(cache, k_new, v_new, &a);
        if (rc != FP4KV_OK)
            return rc;
    }
    Finish f;
    rc = check_finish(a, out, opts, &f);
    if (rc != FP4KV_OK)
        return rc;
    return run_decode(a, f, out, static_cast<hipStream_t>(stream));
}

// The split kernel alone (partials left in the workspace).
int split_call(const fp4kv_cache_layout_t *layout, void *cache, const void *k_new, const void *v_new, bool append,
               const void *q, int32_t batch, int32_t num_q_heads, const int32_t *seq_lens, const int32_t *page_table,
               int32_t max_pages_per_seq, float softmax_scale, int32_t num_splits, void *workspace,
               int64_t workspace_bytes, void *stream)
{
    fp4kv::DecodeArgs a;
    int rc = prepare_split(layout, cache, q, batch, num_q_heads, seq_lens, page_table, max_pages_per_seq,
                           softmax_scale, num_splits, workspace, workspace_bytes, &a);
    if (rc != FP4KV_OK || batch == 0)
        return rc;
    if (append) {
        rc = prepare_append(cache, k_new, v_new, &a);
        if (rc != FP4KV_OK)
            return rc;
    }
    fp4kv::SplitKernel kernel;
    rc = choose_kernel(a, FP4KV_DECODE_KERNEL_AUTO, &kernel);
    if (rc != FP4KV_OK)
        return rc;
    const hipError_t e = fp4kv::launch_decode_split(a, kernel, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP;
}

}  // namespace

extern "C" {

int fp4kv_decode_split(const fp4kv_cache_layout_t *layout, const void *cache, const void *q,
                       int32_t batch, int32_t num_q_heads, const int32_t *seq_lens,
                       const int32_t *page_table, int32_t max_pages_per_seq, float softmax_scale,
                       int32_t num_splits, void *workspace, int64_t workspace_bytes, void *stream)
{
    return split_call(layout, const_cast<void *>(cache), nullptr, nullptr, false, q, batch, num_q_heads, seq_lens,
                      page_table, max_pages_per_seq, softmax_scale, num_splits, workspace, workspace_bytes, stream);
}

int fp4kv_decode_combine(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t partials,
                         const void *workspace, int64_t workspace_bytes, float *out, void *stream)
{
    if (batch < 0 || num_q_heads < 1 || partials < 1)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (head_dim != 64 && head_dim != 128)
        return FP4KV_ERR_UNSUPPORTED;
    if (batch == 0)
        return FP4KV_OK;
    if (!workspace || !out)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, 256) || !aligned(out, 16))
        return FP4KV_ERR_MISALIGNED;
    const int64_t rows = static_cast<int64_t>(batch) * num_q_heads;
    if (rows > std::numeric_limits<int32_t>::max())
        return FP4KV_ERR_UNSUPPORTED;
    const int64_t o_bytes = partial_o_bytes(batch, num_q_heads, partials, head_dim);
    if (workspace_bytes < o_bytes + round_up(rows * partials * 2 * 4, 256))
        return FP4KV_ERR_WORKSPACE_TOO_SMALL;
    const float *ws_o = static_cast<const float *>(workspace);
    const float *ws_ml = reinterpret_cast<const float *>(static_cast<const uint8_t *>(workspace) + o_bytes);
    const hipError_t e = fp4kv::launch_decode_combine(ws_o, ws_ml, batch, num_q_heads, partials, head_dim, out,
                                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP;
}

int fp4kv_decode_attention(const fp4kv_cache_layout_t *layout, const void *cache, const void *q,
                           int32_t batch, int32_t num_q_heads, const int32_t *seq_lens,
                           const int32_t *page_table, int32_t max_pages_per_seq,
                           float softmax_scale, int32_t num_splits, void *workspace,
                           int64_t workspace_bytes, float *out, void *stream)
{
    return decode_call(layout, const_cast<void *>(cache), nullptr, nullptr, false, q, batch, 1, num_q_heads, seq_lens,
                       page_table, max_pages_per_seq, 0, softmax_scale, num_splits, workspace, workspace_bytes, out,
                       nullptr, stream);
}

int fp4kv_decode_attention_noalloc(const fp4kv_cache_layout_t *layout, const void *cache, const void *q,
                                   int32_t batch, int32_t num_q_heads, const int32_t *seq_lens,
                                   const int32_t *page_table, int32_t max_pages_per_seq, float softmax_scale,
                                   int32_t num_splits, float *out, void *stream)
{
    // Every host-visible check runs first, against a stand-in workspace
    // address that is replaced by the static workspace's before any launch;
    // a plan that needs more than the static workspace is rejected here.
    void *const stand_in = reinterpret_cast<void *>(static_cast<uintptr_t>(256));
    fp4kv::DecodeArgs a;
    int rc = prepare_split(layout, cache, q, batch, num_q_heads, seq_lens, page_table, max_pages_per_seq,
                           softmax_scale, num_splits, stand_in, fp4kv::kScratchBytes, &a);
    if (rc != FP4KV_OK || batch == 0)
        return rc;
    Finish f;
    rc = check_finish(a, out, nullptr, &f);
    if (rc != FP4KV_OK)
        return rc;
    void *ws = nullptr;
    if (fp4kv::scratch_for_current_device(&ws) != hipSuccess)
        return FP4KV_ERR_HIP;
    const ptrdiff_t ml_offset = reinterpret_cast<uint8_t *>(a.ws_ml) - static_cast<uint8_t *>(stand_in);
    a.ws_o = static_cast<float *>(ws);
    a.ws_ml = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + ml_offset);
    return run_decode(a, f, out, static_cast<hipStream_t>(stream));
}

int fp4kv_decode_append_split(const fp4kv_cache_layout_t *layout, void *cache, const void *k_new,
                              const void *v_new, const void *q, int32_t batch, int32_t num_q_heads,
                              const int32_t *seq_lens, const int32_t *page_table, int32_t max_pages_per_seq,
                              float softmax_scale, int32_t num_splits, void *workspace, int64_t workspace_bytes,
                              void *stream)
{
    return split_call(layout, cache, k_new, v_new, true, q, batch, num_q_heads, seq_lens, page_table,
                      max_pages_per_seq, softmax_scale, num_splits, workspace, workspace_bytes, stream);
}

int fp4kv_decode_append_attention(const fp4kv_cache_layout_t *layout, void *cache, const void *k_new,
                                  const void *v_new, const void *q, int32_t batch, int32_t num_q_heads,
                                  const int32_t *seq_lens, const int32_t *page_table,
                                  int32_t max_pages_per_seq, float softmax_scale, int32_t num_splits,
                                  void *workspace, int64_t workspace_bytes, float *out, void *stream)
{
    return decode_call(layout, cache, k_new, v_new, true, q, batch, 1, num_q_heads, seq_lens, page_table,
                       max_pages_per_seq, 0, softmax_scale, num_splits, workspace, workspace_bytes, out, nullptr,
                       stream);
}

int fp4kv_decode_multi_attention(const fp4kv_cache_layout_t *layout, const void *cache, const void *q,
                                 int32_t batch, int32_t q_tokens, int32_t num_q_heads, const int32_t *seq_lens,
                                 const int32_t *page_table, int32_t max_pages_per_seq, float softmax_scale,
                                 int32_t num_splits, void *workspace, int64_t workspace_bytes, float *out,
                                 void *stream)
{
    return decode_call(layout, const_cast<void *>(cache), nullptr, nullptr, false, q, batch, q_tokens, num_q_heads,
                       seq_lens, page_table, max_pages_per_seq, 0, softmax_scale, num_splits, workspace,
                       workspace_bytes, out, nullptr, stream);
}

int fp4kv_decode_window_plan(const fp4kv_cache_layout_t *layout, int32_t batch, int32_t q_tokens,
                             int32_t num_q_heads, int32_t max_pages_per_seq, int32_t window, int32_t num_splits,
                             int32_t *splits_out, int32_t *partials_out, int64_t *workspace_bytes_out)
{
    int rc = check_layout(layout);
    if (rc != FP4KV_OK)
        return rc;
    if (!splits_out || !partials_out || !workspace_bytes_out || q_tokens < 1 || window < 0 || num_q_heads < 1 ||
        max_pages_per_seq < 1 || static_cast<int64_t>(q_tokens) * num_q_heads > std::numeric_limits<int32_t>::max())
        return FP4KV_ERR_INVALID_ARGUMENT;
    Plan plan;
    rc = make_plan(*layout, batch, q_tokens * num_q_heads, window_span_pages(max_pages_per_seq, q_tokens, window),
                   num_splits, &plan);
    if (rc != FP4KV_OK)
        return rc;
    *splits_out = plan.splits;
    *partials_out = plan.partials;
    *workspace_bytes_out = plan.ws_bytes;
    return FP4KV_OK;
}

int fp4kv_decode_window_attention(const fp4kv_cache_layout_t *layout, const void *cache, const void *q,
                                  int32_t batch, int32_t q_tokens, int32_t num_q_heads, const int32_t *seq_lens,
                                  const int32_t *page_table, int32_t max_pages_per_seq, int32_t window,
                                  float softmax_scale, int32_t num_splits, void *workspace,
                                  int64_t workspace_bytes, float *out, void *stream)
{
    return decode_call(layout, const_cast<void *>(cache), nullptr, nullptr, false, q, batch, q_tokens, num_q_heads,
                       seq_lens, page_table, max_pages_per_seq, window, softmax_scale, num_splits, workspace,
                       workspace_bytes, out, nullptr, stream);
}

int fp4kv_decode_with_options(const fp4kv_cache_layout_t *layout, void *cache, const void *k_new,
                              const void *v_new, const void *q, int32_t batch, int32_t q_tokens,
                              int32_t num_q_heads, const int32_t *seq_lens, const int32_t *page_table,
                              int32_t max_pages_per_seq, int32_t window, float softmax_scale, int32_t num_splits,
                              void *workspace, int64_t workspace_bytes, float *out,
                              const fp4kv_decode_options *options, void *stream)
{
    const bool append = k_new || v_new;
    if (append && (q_tokens != 1 || window != 0))
        return FP4KV_ERR_UNSUPPORTED;
    return decode_call(layout, cache, k_new, v_new, append, q, batch, q_tokens, num_q_heads, seq_lens, page_table,
                       max_pages_per_seq, window, softmax_scale, num_splits, workspace, workspace_bytes, out, options,
                       stream);
}

const char *fp4kv_status_string(int status)
{
    switch (status) {
    case FP4KV_OK: return "ok";
    case FP4KV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FP4KV_ERR_UNSUPPORTED: return "unsupported shape";
    case FP4KV_ERR_MISALIGNED: return "misaligned pointer";
    case FP4KV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FP4KV_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
    }
}

int fp4kv_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *stream)
{
    constexpr int64_t kBlock = 9216;
    if (!buf || !sink || bytes <= 0 || bytes % kBlock != 0)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (!aligned(buf, 256) || !aligned(sink, 4))
        return FP4KV_ERR_MISALIGNED;
    const hipError_t e = fp4kv::launch_read_probe(static_cast<const uint8_t *>(buf), bytes / kBlock, sink,
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP;
}

int fp4kv_read_probe_config(const void *buf, int64_t bytes, int32_t loads_per_lane, int32_t workgroups,
                            int32_t to_lds, uint32_t *sink, void *stream)
{
    if (!buf || !sink || bytes <= 0 || workgroups < 1 || (to_lds != 0 && to_lds != 1))
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8 &&
        loads_per_lane != 16)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (bytes % (1024 * static_cast<int64_t>(loads_per_lane)) != 0)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (!aligned(buf, 1024) || !aligned(sink, 4))
        return FP4KV_ERR_MISALIGNED;
    const hipError_t e = fp4kv::launch_read_probe_config(static_cast<const uint8_t *>(buf), bytes, loads_per_lane,
                                                         workgroups, to_lds != 0, sink,
                                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP;
}

int fp4kv_stream_probe(const void *src, void *dst, int64_t units, int32_t read_bytes, int32_t write_bytes,
                       int32_t paired, int32_t workgroups, uint32_t *sink, void *stream)
{
    if (!src || !sink || units < 1 || read_bytes < 8192 || read_bytes % 8192 != 0 || write_bytes < 0 ||
        write_bytes % 1024 != 0 || (write_bytes > 0 && !dst) || workgroups < 1 || (paired != 0 && paired != 1))
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (!aligned(src, 1024) || (dst && !aligned(dst, 1024)) || !aligned(sink, 4))
        return FP4KV_ERR_MISALIGNED;
    const hipError_t e = fp4kv::launch_stream_probe(static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), units,
                                                    read_bytes, write_bytes, paired != 0, workgroups, sink,
                                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP;
}

int fp4kv_version(void) { return FP4KV_VERSION; }

}  // extern "C"
