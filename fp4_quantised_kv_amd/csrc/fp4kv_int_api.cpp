// Host side of the integer-format C ABI (include/fp4kv_int.h): sizes,
// argument checks, split planning and launches.  Every check runs before the
// first HIP call.
#include "fp4kv_int.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>

#include <hip/hip_runtime.h>

#include "fp4kv_internal.h"

namespace {

constexpr int64_t kChunk = 256;          // tokens per split unit
constexpr int64_t kTargetGroups = 2048;  // workgroups the automatic split count aims at
constexpr int64_t kMaxSplits = 65535;    // the split kernel's third grid dimension

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
bool known_bits(int32_t bits)
{
    return bits == 2 || bits == 4 || bits == 8 || bits == 16 || bits == FP4KV_INT_FP8_E4M3;
}
// bits per stored element
int32_t element_bits(int32_t bits) { return bits == FP4KV_INT_FP8_E4M3 ? 8 : bits; }
bool known_granularity(int32_t g) { return g == FP4KV_INT_PER_TOKEN || g == FP4KV_INT_PER_CHANNEL; }

int check_dims(const fp4kv_int_dims *d)
{
    if (!d || d->batch < 0 || d->tokens < 0 || d->num_kv_heads < 1)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (d->head_dim != 64 && d->head_dim != 128)
        return FP4KV_ERR_UNSUPPORTED;
    return FP4KV_OK;
}

struct IntSizes {
    int64_t code_bytes, scale_bytes;
};

int sizes_of(const fp4kv_int_dims &d, int32_t bits, int32_t granularity, IntSizes *out)
{
    if (!known_bits(bits) || !known_granularity(granularity))
        return FP4KV_ERR_INVALID_ARGUMENT;
    const int64_t rows = static_cast<int64_t>(d.batch) * d.tokens * d.num_kv_heads;
    const int64_t row_bytes = static_cast<int64_t>(d.head_dim) * element_bits(bits) / 8;
    if (rows > std::numeric_limits<int64_t>::max() / 2 / row_bytes)
        return FP4KV_ERR_INVALID_ARGUMENT;
    out->code_bytes = rows * row_bytes;
    if (bits == 16)
        out->scale_bytes = 0;
    else if (granularity == FP4KV_INT_PER_TOKEN)
        out->scale_bytes = rows * 2;
    else
        out->scale_bytes = static_cast<int64_t>(d.batch) * d.num_kv_heads * d.head_dim * 2;
    return FP4KV_OK;
}

struct IntPlan {
    int32_t splits, chunks_per_split;
    int64_t ws_o_bytes, ws_bytes;
};

int plan_of(const fp4kv_int_dims &d, int32_t num_q_heads, int32_t num_splits, IntPlan *out)
{
    if (num_q_heads < 1 || num_splits < 0 || num_q_heads % d.num_kv_heads)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (num_q_heads / d.num_kv_heads > FP4KV_MAX_GROUP)
        return FP4KV_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(d.batch) > 65535 || d.num_kv_heads > 65535)
        return FP4KV_ERR_UNSUPPORTED;
    const int64_t chunks = (static_cast<int64_t>(d.tokens) + kChunk - 1) / kChunk;
    int64_t want = num_splits;
    if (want == 0) {
        const int64_t per_split = std::max<int64_t>(1, static_cast<int64_t>(d.batch) * d.num_kv_heads);
        want = (kTargetGroups + per_split - 1) / per_split;
    }
    want = std::min<int64_t>(want, std::max<int64_t>(chunks, 1));
    want = std::min<int64_t>(want, kMaxSplits);
    const int64_t cps = chunks ? (chunks + want - 1) / want : 1;
    const int64_t splits = chunks ? (chunks + cps - 1) / cps : 1;   // no split starts past the end
    const int64_t rows = static_cast<int64_t>(d.batch) * num_q_heads * splits;
    out->splits = static_cast<int32_t>(splits);
    out->chunks_per_split = static_cast<int32_t>(cps);
    out->ws_o_bytes = round_up(rows * d.head_dim * 4, 256);
    out->ws_bytes = out->ws_o_bytes + round_up(rows * 2 * 4, 256);
    return FP4KV_OK;
}

}  // namespace

extern "C" {

int fp4kv_int_sizes(const fp4kv_int_dims *dims, int32_t bits, int32_t granularity, int64_t *code_bytes_out,
                    int64_t *scale_bytes_out)
{
    int rc = check_dims(dims);
    if (rc != FP4KV_OK)
        return rc;
    if (!code_bytes_out || !scale_bytes_out)
        return FP4KV_ERR_INVALID_ARGUMENT;
    IntSizes s;
    rc = sizes_of(*dims, bits, granularity, &s);
    if (rc != FP4KV_OK)
        return rc;
    *code_bytes_out = s.code_bytes;
    *scale_bytes_out = s.scale_bytes;
    return FP4KV_OK;
}

int fp4kv_int_quantize(const fp4kv_int_dims *dims, int32_t bits, int32_t granularity, const void *x,
                       void *codes, void *scales, void *stream)
{
    int rc = check_dims(dims);
    if (rc != FP4KV_OK)
        return rc;
    IntSizes s;
    rc = sizes_of(*dims, bits, granularity, &s);
    if (rc != FP4KV_OK)
        return rc;
    if (s.code_bytes == 0)
        return FP4KV_OK;
    if (!x || !codes || (bits != 16 && !scales))
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (!aligned(x, 16) || !aligned(codes, 16) || (bits != 16 && !aligned(scales, 16)))
        return FP4KV_ERR_MISALIGNED;
    const int64_t threads =
        s.code_bytes / (static_cast<int64_t>(dims->head_dim) * element_bits(bits) / 8) * (dims->head_dim / 16);
    if ((threads + 255) / 256 > std::numeric_limits<int32_t>::max())
        return FP4KV_ERR_UNSUPPORTED;
    if (bits != 16 && granularity == FP4KV_INT_PER_CHANNEL && dims->batch > 65535)
        return FP4KV_ERR_UNSUPPORTED;
    fp4kv::IntQuantArgs q{};
    q.x = static_cast<const uint16_t *>(x);
    q.codes = static_cast<uint8_t *>(codes);
    q.scales = static_cast<uint16_t *>(scales);
    q.batch = dims->batch;
    q.tokens = dims->tokens;
    q.num_kv_heads = dims->num_kv_heads;
    q.head_dim = dims->head_dim;
    q.bits = bits;
    q.per_channel = granularity == FP4KV_INT_PER_CHANNEL;
    const hipError_t e = fp4kv::launch_int_quantize(q, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP;
}

int fp4kv_int_decode_plan(const fp4kv_int_dims *dims, int32_t num_q_heads, int32_t num_splits,
                          int32_t *splits_out, int64_t *workspace_bytes_out)
{
    int rc = check_dims(dims);
    if (rc != FP4KV_OK)
        return rc;
    if (!splits_out || !workspace_bytes_out)
        return FP4KV_ERR_INVALID_ARGUMENT;
    IntPlan p;
    rc = plan_of(*dims, num_q_heads, num_splits, &p);
    if (rc != FP4KV_OK)
        return rc;
    *splits_out = p.splits;
    *workspace_bytes_out = p.ws_bytes;
    return FP4KV_OK;
}

int fp4kv_int_decode_attention(const fp4kv_int_dims *dims, int32_t bits, int32_t k_granularity,
                               int32_t v_granularity, const void *k_codes, const void *k_scales,
                               const void *v_codes, const void *v_scales, const void *q,
                               int32_t num_q_heads, float softmax_scale, int32_t num_splits,
                               void *workspace, int64_t workspace_bytes, float *out, void *stream)
{
    int rc = check_dims(dims);
    if (rc != FP4KV_OK)
        return rc;
    IntSizes ks, vs;
    if ((rc = sizes_of(*dims, bits, k_granularity, &ks)) != FP4KV_OK ||
        (rc = sizes_of(*dims, bits, v_granularity, &vs)) != FP4KV_OK)
        return rc;
    IntPlan p;
    rc = plan_of(*dims, num_q_heads, num_splits, &p);
    if (rc != FP4KV_OK)
        return rc;
    if (!(std::isfinite(softmax_scale) && softmax_scale > 0.0f))
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (dims->batch == 0)
        return FP4KV_OK;
    if (!q || !out || !workspace)
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (dims->tokens > 0 && (!k_codes || !v_codes || (bits != 16 && (!k_scales || !v_scales))))
        return FP4KV_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(workspace, 256) || !aligned(k_codes, 16) ||
        !aligned(v_codes, 16) || !aligned(k_scales, 2) || !aligned(v_scales, 2))
        return FP4KV_ERR_MISALIGNED;
    if (workspace_bytes < p.ws_bytes)
        return FP4KV_ERR_WORKSPACE_TOO_SMALL;
    fp4kv::IntDecodeArgs a{};
    a.k_codes = static_cast<const uint8_t *>(k_codes);
    a.v_codes = static_cast<const uint8_t *>(v_codes);
    a.k_scales = static_cast<const uint16_t *>(k_scales);
    a.v_scales = static_cast<const uint16_t *>(v_scales);
    a.q = static_cast<const uint16_t *>(q);
    a.tokens = dims->tokens;
    a.batch = dims->batch;
    a.num_kv_heads = dims->num_kv_heads;
    a.num_q_heads = num_q_heads;
    a.group = num_q_heads / dims->num_kv_heads;
    a.head_dim = dims->head_dim;
    a.bits = bits;
    a.splits = p.splits;
    a.chunks_per_split = p.chunks_per_split;
    a.k_per_channel = bits != 16 && k_granularity == FP4KV_INT_PER_CHANNEL;
    a.v_per_channel = bits != 16 && v_granularity == FP4KV_INT_PER_CHANNEL;
    a.scale_log2e = softmax_scale * 1.4426950408889634f;
    a.ws_o = static_cast<float *>(workspace);
    a.ws_ml = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + p.ws_o_bytes);
    a.out = out;
    const hipError_t e = fp4kv::launch_int_decode(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP;
}

}  // extern "C"
