// Host-only stand-ins for the library's kernel launchers, so that the C ABI's
// host code (argument checks, plans, chunk sizes, workspace carving) can be
// built and run under AddressSanitizer and UndefinedBehaviorSanitizer on a
// machine without a GPU.  Each stub checks the invariants its real kernel
// relies on and counts its calls; none touches the (fake) device pointers.
#include <cstdio>
#include <cstdlib>

#include "fp4kv_internal.h"

namespace fp4kv {

int g_stub_calls = 0;

static void require(bool ok, const char *what)
{
    if (!ok) {
        std::fprintf(stderr, "stub invariant failed: %s\n", what);
        std::abort();
    }
}

static void check_split(const DecodeArgs &a)
{
    require(a.cache && a.q && a.seq_lens && a.page_table && a.ws_o && a.ws_ml, "decode pointers");
    require(a.batch >= 1 && a.group >= 1 && a.partials >= 1 && a.pages_per_split >= 1, "decode sizes");
    const int64_t chunks = static_cast<int64_t>(a.partials) * 4;
    require(a.lead_chunks >= 0 && a.lead_chunks <= chunks && a.lead_pages >= 1 && a.tail_pages >= 1, "chunk sizes");
    const int64_t covered = static_cast<int64_t>(a.lead_chunks) * a.lead_pages + (chunks - a.lead_chunks) * a.tail_pages;
    // the chunks tile the span the plan was made for (the whole table without a window)
    require(a.window > 0 || covered >= a.max_pages, "chunks cover the table");
    require(!a.k_new == !a.v_new && !a.k_new == !a.cache_w, "append pointers");
}

hipError_t launch_quantize_append(const CacheGeom &g, const uint16_t *k, const uint16_t *v, int64_t n_tokens,
                                  const int64_t *slots, uint8_t *cache, hipStream_t)
{
    require(n_tokens > 0 && k && v && slots && cache && g.num_pages >= 1, "append arguments");
    ++g_stub_calls;
    return hipSuccess;
}

hipError_t launch_split_valu(const DecodeArgs &a, hipStream_t) { check_split(a); ++g_stub_calls; return hipSuccess; }
hipError_t launch_split_mfma(const DecodeArgs &a, hipStream_t) { check_split(a); ++g_stub_calls; return hipSuccess; }
hipError_t launch_split_fp8(const DecodeArgs &a, hipStream_t) { check_split(a); ++g_stub_calls; return hipSuccess; }

hipError_t launch_decode_split(const DecodeArgs &a, SplitKernel, hipStream_t)
{
    check_split(a);
    ++g_stub_calls;
    return hipSuccess;
}

hipError_t launch_append_last(const DecodeArgs &a, hipStream_t) { check_split(a); ++g_stub_calls; return hipSuccess; }

bool split_appends_itself(SplitKernel kernel) { return kernel == SplitKernel::mfma_staged || kernel == SplitKernel::fp8; }

hipError_t launch_decode_combine(const float *ws_o, const float *ws_ml, int32_t batch, int32_t num_q_heads,
                                 int32_t partials, int32_t head_dim, float *out, hipStream_t)
{
    require(ws_o && ws_ml && out && batch >= 1 && num_q_heads >= 1 && partials >= 1, "combine arguments");
    require(head_dim == 64 || head_dim == 128, "combine head size");
    ++g_stub_calls;
    return hipSuccess;
}

static uint8_t g_fake_scratch alignas(256)[256];

hipError_t scratch_for_current_device(void **out)
{
    *out = g_fake_scratch;
    return hipSuccess;
}

hipError_t launch_read_probe(const uint8_t *buf, int64_t blocks, uint32_t *sink, hipStream_t)
{
    require(buf && sink && blocks > 0, "read probe");
    ++g_stub_calls;
    return hipSuccess;
}

hipError_t launch_stream_probe(const uint8_t *src, uint8_t *, int64_t units, int read_bytes, int write_bytes, bool,
                               int workgroups, uint32_t *sink, hipStream_t)
{
    require(src && sink && units > 0 && read_bytes % 8192 == 0 && write_bytes % 1024 == 0 && workgroups > 0,
            "stream probe");
    ++g_stub_calls;
    return hipSuccess;
}

hipError_t launch_read_probe_config(const uint8_t *buf, int64_t bytes, int loads_per_lane, int workgroups, bool,
                                    uint32_t *sink, hipStream_t)
{
    require(buf && sink && bytes % (1024 * loads_per_lane) == 0 && workgroups > 0, "read probe config");
    ++g_stub_calls;
    return hipSuccess;
}

hipError_t launch_int_quantize(const IntQuantArgs &, hipStream_t) { ++g_stub_calls; return hipSuccess; }
hipError_t launch_int_decode(const IntDecodeArgs &, hipStream_t) { ++g_stub_calls; return hipSuccess; }

}  // namespace fp4kv
