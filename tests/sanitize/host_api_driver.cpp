// Drives every entry point of include/fp4kv.h and include/fp4kv_int.h with
// valid and invalid host arguments, linked against launch_stubs.cpp instead
// of the kernels, under AddressSanitizer and UndefinedBehaviorSanitizer.
// Device pointers are fake, aligned addresses: the host code only checks and
// forwards them.  Prints "ok" and exits 0 when every expectation holds.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <limits>

#include "fp4kv.h"
#include "fp4kv_int.h"

namespace fp4kv {
extern int g_stub_calls;
}

static int g_failures = 0;

#define EXPECT(cond)                                                                      \
    do {                                                                                  \
        if (!(cond)) {                                                                    \
            std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_failures;                                                                 \
        }                                                                                 \
    } while (0)

static void *dev(uintptr_t mb) { return reinterpret_cast<void *>(mb << 20); }   // 1 MB aligned fake address

static fp4kv_cache_layout_t layout(int32_t H, int32_t D, int64_t pages, int32_t format = FP4KV_FORMAT_FP4_E2M1)
{
    fp4kv_cache_params p{H, D, FP4KV_PAGE_SIZE, format, pages, 0.0f, 0.0f};
    if (format == FP4KV_FORMAT_FP8_E4M3)
        p.k_scale = p.v_scale = 0.5f;
    fp4kv_cache_layout_t L;
    std::memset(&L, 0, sizeof L);
    EXPECT(fp4kv_cache_layout(&p, &L) == FP4KV_OK);
    return L;
}

static void layouts()
{
    for (int32_t f : {int32_t(FP4KV_FORMAT_FP4_E2M1), int32_t(FP4KV_FORMAT_FP8_E4M3), int32_t(FP4KV_FORMAT_FP8_E4M3_TOKEN)})
        for (int32_t D : {64, 128})
            for (int32_t H : {1, 3, 8, 64})
                for (int64_t pages : {int64_t(1), int64_t(1000), int64_t(1) << 24}) {
                    const fp4kv_cache_layout_t L = layout(H, D, pages, f);
                    EXPECT(L.cache_bytes == pages * L.page_stride && L.page_stride == H * L.block_bytes);
                }
    fp4kv_cache_layout_t L;
    fp4kv_cache_params bad[] = {
        {0, 128, 64, 0, 1, 0, 0},  {8, 96, 64, 0, 1, 0, 0},   {8, 128, 32, 0, 1, 0, 0},
        {8, 128, 64, 7, 1, 0, 0},  {8, 128, 64, 0, 0, 0, 0},  {8, 128, 64, 0, int64_t(1) << 60, 0, 0},
        {8, 128, 64, 1, 1, 0, 1},  {8, 128, 64, 1, 1, std::numeric_limits<float>::infinity(), 1},
        {8, 128, 64, 1, 1, std::numeric_limits<float>::quiet_NaN(), 1}, {8, 128, 64, 2, 1, 1, 0},
        {std::numeric_limits<int32_t>::max(), 128, 64, 0, std::numeric_limits<int64_t>::max(), 0, 0},
    };
    for (const auto &p : bad)
        EXPECT(fp4kv_cache_layout(&p, &L) != FP4KV_OK);
    EXPECT(fp4kv_cache_layout(nullptr, &L) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_cache_layout(&bad[0], nullptr) == FP4KV_ERR_INVALID_ARGUMENT);
    for (int s = -10; s <= 2; ++s)
        EXPECT(fp4kv_status_string(s) != nullptr);
    EXPECT(fp4kv_version() == FP4KV_VERSION);
}

static void plans()
{
    const fp4kv_cache_layout_t L = layout(8, 128, 32 * 512);
    int32_t s, p, lc, lp, tp;
    int64_t ws;
    for (int32_t B : {0, 1, 7, 32, 64, 65535})
        for (int32_t maxp : {1, 2, 9, 257, 512, 8192, 1 << 20})
            for (int32_t S : {0, 1, 3, 64, 256, 1000, 1 << 20})
                for (int32_t qt : {1, 2, 16})
                    for (int32_t win : {0, 1, 700, 1 << 20})
                        for (int32_t min_len : {0, 1, maxp * 32, maxp * 64}) {
                            const int rc = fp4kv_decode_chunks(&L, B, qt, 32 * (qt == 16 ? 1 : 8 / qt), maxp, win, S,
                                                               min_len, &lc, &lp, &tp);
                            if (rc != FP4KV_OK)
                                continue;
                            EXPECT(lc >= 1 && lp >= 1 && tp >= 1 && tp <= lp);
                            if (win == 0 && qt == 1) {
                                EXPECT(fp4kv_decode_plan(&L, B, 64, maxp, S, &s, &p, &ws) == FP4KV_OK);
                                EXPECT(int64_t(lc) * lp + int64_t(4 * p - lc) * tp >= maxp);
                            }
                        }
    EXPECT(fp4kv_decode_plan(&L, 32, 64, 512, 64, &s, &p, &ws) == FP4KV_OK && s == 64 && p == 16);
    EXPECT(fp4kv_decode_chunks(&L, 32, 1, 64, 512, 0, 64, 0, &lc, &lp, &tp) == FP4KV_OK && lc == 32 && lp == 13 &&
           tp == 3);
    EXPECT(fp4kv_decode_chunks(&L, 32, 1, 64, 512, 0, 64, 32768, &lc, &lp, &tp) == FP4KV_OK && lc == 12 &&
           lp == 39 && tp == 1);
    EXPECT(fp4kv_decode_plan(&L, -1, 64, 512, 64, &s, &p, &ws) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_plan(&L, 1, 65, 512, 64, &s, &p, &ws) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_plan(&L, 1, 64, 512, 64, nullptr, &p, &ws) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_plan(nullptr, 1, 64, 512, 64, &s, &p, &ws) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_chunks(&L, 1, 0, 64, 512, 0, 64, 0, &lc, &lp, &tp) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_chunks(&L, 1, 1, 64, 512, -1, 64, 0, &lc, &lp, &tp) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_chunks(&L, 1, 1, 64, 512, 0, 64, -1, &lc, &lp, &tp) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_window_plan(&L, 4, 2, 64, 100, 700, 0, &s, &p, &ws) == FP4KV_OK);
    EXPECT(fp4kv_decode_window_plan(&L, 4, 0, 64, 100, 700, 0, &s, &p, &ws) != FP4KV_OK);
}

static void decode_calls()
{
    const fp4kv_cache_layout_t L = layout(8, 128, 32 * 512);
    int32_t s, p;
    int64_t ws;
    EXPECT(fp4kv_decode_plan(&L, 32, 64, 512, 64, &s, &p, &ws) == FP4KV_OK);
    const auto lens = static_cast<const int32_t *>(dev(3));
    const auto table = static_cast<const int32_t *>(dev(4));
    float *out = static_cast<float *>(dev(5));
    const int before = fp4kv::g_stub_calls;
    EXPECT(fp4kv_decode_attention(&L, dev(1), dev(2), 32, 64, lens, table, 512, 0.088f, 64, dev(6), ws, out,
                                  nullptr) == FP4KV_OK);
    EXPECT(fp4kv::g_stub_calls == before + 2);                   // split + combine
    EXPECT(fp4kv_decode_split(&L, dev(1), dev(2), 32, 64, lens, table, 512, 0.088f, 64, dev(6), ws, nullptr) ==
           FP4KV_OK);
    EXPECT(fp4kv_decode_combine(32, 64, 128, p, dev(6), ws, out, nullptr) == FP4KV_OK);
    EXPECT(fp4kv_decode_append_attention(&L, dev(1), dev(7), dev(8), dev(2), 32, 64, lens, table, 512, 0.088f, 64,
                                         dev(6), ws, out, nullptr) == FP4KV_OK);
    EXPECT(fp4kv_decode_append_split(&L, dev(1), dev(7), dev(8), dev(2), 32, 64, lens, table, 512, 0.088f, 64,
                                     dev(6), ws, nullptr) == FP4KV_OK);
    EXPECT(fp4kv_decode_attention_noalloc(&L, dev(1), dev(2), 32, 64, lens, table, 512, 0.088f, 64, out,
                                          nullptr) == FP4KV_OK);
    int64_t wsm;
    EXPECT(fp4kv_decode_window_plan(&L, 32, 2, 32, 512, 0, 0, &s, &p, &wsm) == FP4KV_OK);
    EXPECT(fp4kv_decode_multi_attention(&L, dev(1), dev(2), 32, 2, 32, lens, table, 512, 0.088f, 0, dev(6), wsm,
                                        out, nullptr) == FP4KV_OK);
    EXPECT(fp4kv_decode_window_plan(&L, 32, 2, 32, 512, 700, 0, &s, &p, &wsm) == FP4KV_OK);
    EXPECT(fp4kv_decode_window_attention(&L, dev(1), dev(2), 32, 2, 32, lens, table, 512, 700, 0.088f, 0, dev(6),
                                         wsm, out, nullptr) == FP4KV_OK);
    for (int32_t k : {0, 1, 2, 3})
        for (int32_t m : {0, 1})
            for (int32_t min_len : {0, 32768}) {
                const fp4kv_decode_options o{k, m, min_len};
                EXPECT(fp4kv_decode_with_options(&L, dev(1), nullptr, nullptr, dev(2), 32, 1, 64, lens, table, 512, 0,
                                                 0.088f, 64, dev(6), ws, out, &o, nullptr) == FP4KV_OK);
            }
    {
        // the split kernel alone: one launch, no output pointer needed
        const fp4kv_decode_options o{0, 2, 32768};
        const int before_split = fp4kv::g_stub_calls;
        EXPECT(fp4kv_decode_with_options(&L, dev(1), nullptr, nullptr, dev(2), 32, 1, 64, lens, table, 512, 0,
                                         0.088f, 64, dev(6), ws, nullptr, &o, nullptr) == FP4KV_OK);
        EXPECT(fp4kv::g_stub_calls == before_split + 1);
    }
    const fp4kv_decode_options bad_kernel{9, 0, 0}, bad_merge{0, 9, 0}, bad_min{0, 0, -1};
    EXPECT(fp4kv_decode_with_options(&L, dev(1), nullptr, nullptr, dev(2), 32, 1, 64, lens, table, 512, 0, 0.088f,
                                     64, dev(6), ws, out, &bad_min, nullptr) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_with_options(&L, dev(1), nullptr, nullptr, dev(2), 32, 1, 64, lens, table, 512, 0, 0.088f,
                                     64, dev(6), ws, out, &bad_kernel, nullptr) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_with_options(&L, dev(1), nullptr, nullptr, dev(2), 32, 1, 64, lens, table, 512, 0, 0.088f,
                                     64, dev(6), ws, out, &bad_merge, nullptr) == FP4KV_ERR_INVALID_ARGUMENT);
    // refusals before any launch
    const int n = fp4kv::g_stub_calls;
    EXPECT(fp4kv_decode_attention(&L, dev(1), dev(2), 32, 64, lens, table, 512, 0.088f, 64, dev(6), ws - 1, out,
                                  nullptr) == FP4KV_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(fp4kv_decode_attention(&L, dev(1), dev(2), 32, 64, lens, table, 512, -1.0f, 64, dev(6), ws, out,
                                  nullptr) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_attention(&L, dev(1), dev(2), 32, 64, lens, table, 512,
                                  std::numeric_limits<float>::quiet_NaN(), 64, dev(6), ws, out, nullptr) ==
           FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_attention(&L, static_cast<char *>(dev(1)) + 8, dev(2), 32, 64, lens, table, 512, 0.088f, 64,
                                  dev(6), ws, out, nullptr) == FP4KV_ERR_MISALIGNED);
    EXPECT(fp4kv_decode_attention(&L, dev(1), dev(2), 32, 64, nullptr, table, 512, 0.088f, 64, dev(6), ws, out,
                                  nullptr) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_attention(&L, dev(1), dev(2), 32, 64 * 17, lens, table, 512, 0.088f, 64, dev(6), ws, out,
                                  nullptr) != FP4KV_OK);
    EXPECT(fp4kv_decode_append_attention(&L, dev(1), nullptr, dev(8), dev(2), 32, 64, lens, table, 512, 0.088f, 64,
                                         dev(6), ws, out, nullptr) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_window_attention(&L, dev(1), dev(2), 32, 2, 32, lens, table, 512, -1, 0.088f, 0, dev(6),
                                         wsm, out, nullptr) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_decode_combine(32, 64, 96, 16, dev(6), ws, out, nullptr) != FP4KV_OK);
    EXPECT(fp4kv::g_stub_calls == n);
    // batch 0 is a no-op
    EXPECT(fp4kv_decode_attention(&L, nullptr, nullptr, 0, 64, nullptr, nullptr, 512, 0.088f, 0, nullptr, 0, out,
                                  nullptr) == FP4KV_OK);
}

static void appends_and_probes()
{
    const fp4kv_cache_layout_t L = layout(8, 128, 100);
    const auto slots = static_cast<const int64_t *>(dev(3));
    EXPECT(fp4kv_quantize_append(&L, dev(1), dev(2), 1000, slots, dev(4), nullptr) == FP4KV_OK);
    EXPECT(fp4kv_quantize_append(&L, dev(1), dev(2), 0, slots, dev(4), nullptr) == FP4KV_OK);
    EXPECT(fp4kv_quantize_append(&L, dev(1), dev(2), -1, slots, dev(4), nullptr) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_quantize_append(&L, nullptr, dev(2), 5, slots, dev(4), nullptr) == FP4KV_ERR_INVALID_ARGUMENT);
    EXPECT(fp4kv_quantize_append(&L, static_cast<char *>(dev(1)) + 2, dev(2), 5, slots, dev(4), nullptr) ==
           FP4KV_ERR_MISALIGNED);
    auto sink = static_cast<uint32_t *>(dev(9));
    EXPECT(fp4kv_read_probe(dev(1), 9216 * 10, sink, nullptr) == FP4KV_OK);
    EXPECT(fp4kv_read_probe(dev(1), 9215, sink, nullptr) != FP4KV_OK);
    for (int32_t loads : {1, 2, 4, 8, 16})
        EXPECT(fp4kv_read_probe_config(dev(1), 16384 * 4, loads, 512, loads & 1, sink, nullptr) == FP4KV_OK);
    EXPECT(fp4kv_read_probe_config(dev(1), 16384, 3, 512, 0, sink, nullptr) != FP4KV_OK);
    EXPECT(fp4kv_stream_probe(dev(1), dev(2), 10, 65536, 18432, 1, 1024, sink, nullptr) == FP4KV_OK);
    EXPECT(fp4kv_stream_probe(dev(1), nullptr, 10, 65536, 0, 0, 1024, sink, nullptr) == FP4KV_OK);
    EXPECT(fp4kv_stream_probe(dev(1), dev(2), 10, 65536, 1000, 0, 1024, sink, nullptr) != FP4KV_OK);
}

static void int_formats()
{
    int64_t cb, sb, ws;
    int32_t s;
    for (int32_t bits : {2, 4, 8, 16, static_cast<int32_t>(FP4KV_INT_FP8_E4M3)})
        for (int32_t gran : {static_cast<int32_t>(FP4KV_INT_PER_TOKEN), static_cast<int32_t>(FP4KV_INT_PER_CHANNEL)})
            for (int32_t D : {64, 128}) {
                const fp4kv_int_dims d{4, 300, 8, D};
                if (fp4kv_int_sizes(&d, bits, gran, &cb, &sb) != FP4KV_OK)
                    continue;
                EXPECT(cb > 0 && sb >= 0);
                EXPECT(fp4kv_int_quantize(&d, bits, gran, dev(1), dev(2), dev(3), nullptr) == FP4KV_OK);
                EXPECT(fp4kv_int_decode_plan(&d, 32, 0, &s, &ws) == FP4KV_OK);
                EXPECT(fp4kv_int_decode_attention(&d, bits, gran, gran, dev(2), dev(3), dev(4), dev(5), dev(6), 32,
                                                  0.088f, 0, dev(7), ws, static_cast<float *>(dev(8)),
                                                  nullptr) == FP4KV_OK);
            }
    const fp4kv_int_dims bad{-1, 300, 8, 128};
    EXPECT(fp4kv_int_sizes(&bad, 4, 0, &cb, &sb) != FP4KV_OK);
    const fp4kv_int_dims d{4, 300, 8, 128};
    EXPECT(fp4kv_int_sizes(&d, 3, 0, &cb, &sb) != FP4KV_OK);
    EXPECT(fp4kv_int_sizes(&d, 4, 7, &cb, &sb) != FP4KV_OK);
    EXPECT(fp4kv_int_sizes(nullptr, 4, 0, &cb, &sb) != FP4KV_OK);
}

int main()
{
    layouts();
    plans();
    decode_calls();
    appends_and_probes();
    int_formats();
    if (g_failures) {
        std::fprintf(stderr, "%d expectations failed\n", g_failures);
        return 1;
    }
    std::printf("ok: %d launches stubbed\n", fp4kv::g_stub_calls);
    return 0;
}
