// Internal interface between the host API (fp4kv_api.cpp) and the HIP kernels
// (fp4kv_kernels.hip).  Not installed; the public ABI is include/fp4kv.h.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace fp4kv {

// Cache geometry, copied out of a validated fp4kv_cache_layout_t.
struct CacheGeom {
    int32_t num_kv_heads;
    int32_t head_dim;
    int64_t num_pages;
    int64_t k_codes_off, k_scales_off, v_codes_off, v_scales_off;
    int64_t head_stride, page_stride;
    bool fp8;                    // FP8 E4M3 elements (else FP4)
    bool token_scales;           // FP8 with an fp16 scale per (token, KV head) (else per tensor)
    float k_scale, v_scale;      // FP8 per-tensor scales
};

struct DecodeArgs {
    CacheGeom geom;
    const uint8_t *cache;
    const uint16_t *q;           // bf16 [batch][q_tokens][num_q_heads][D]
    const int32_t *seq_lens;     // [batch]
    const int32_t *page_table;   // [batch][max_pages]
    int32_t batch, num_q_heads, group, max_pages;
    int32_t q_tokens;            // query tokens per sequence (1: plain decode); q_tokens * group <= 16
    int32_t window;              // > 0: a query sees only the last `window` tokens of its prefix (sliding window)
    int32_t splits, pages_per_split;   // context chunks and pages per chunk (from the window's first page)
    int32_t partials;            // partial slots per row: ceil(splits / 4), one per workgroup
    // Chunk sizes (pages): the first lead_chunks chunks hold lead_pages
    // each, the rest tail_pages each (all pages_per_split: even chunks)
    int32_t lead_chunks, lead_pages, tail_pages;
    float scale_log2e;           // softmax scale times log2(e): scores kept in base 2
    float *ws_o;                 // [batch][partials][q_tokens * num_q_heads][D] unnormalised outputs
    float *ws_ml;                // [batch][partials][q_tokens * num_q_heads][2] running max (base 2), sum
    float *out;                  // [batch][q_tokens * num_q_heads][D]; set only with one partial per
                                 // row: the split kernel then writes the final rows, no combine
    bool staged;                 // matrix-core kernel: stage pages through LDS (D = 128)
    // The step's own token, appended before attending (all null: no append):
    // bf16 K and V rows [batch][H_kv][D] of one token per sequence, placed at
    // position seq_lens[b] - 1 through the page table, in the cache at cache_w
    // (the same bytes as `cache`).
    const uint16_t *k_new, *v_new;
    uint8_t *cache_w;
};

hipError_t launch_quantize_append(const CacheGeom &g, const uint16_t *k, const uint16_t *v,
                                  int64_t n_tokens, const int64_t *slots, uint8_t *cache,
                                  hipStream_t stream);

// Decode split kernels: the vector-ALU one and the matrix-core one.
hipError_t launch_split_valu(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_split_mfma(const DecodeArgs &a, hipStream_t stream);
// The FP8 cache's kernel (D = 128).
hipError_t launch_split_fp8(const DecodeArgs &a, hipStream_t stream);

// The split kernel of a decode call, chosen once per call by the host API:
// the FP8 kernel for an FP8 cache; for FP4 the matrix-core kernel with LDS
// staging (D = 128), the matrix-core kernel with operands loaded straight
// into registers (any D; the D = 64 kernel), or the vector-ALU kernel (one
// query token, no window).
enum class SplitKernel { fp8, mfma_staged, mfma_direct, valu };

// Launches the chosen split kernel, preceded by the append kernel when the
// call appends the step's token (a.k_new set) and that kernel does not store
// it itself.
hipError_t launch_decode_split(const DecodeArgs &a, SplitKernel kernel, hipStream_t stream);

// Places each sequence's k_new / v_new row at position seq_lens[b] - 1 (a
// kernel of its own, for the decode kernels that do not append themselves).
hipError_t launch_append_last(const DecodeArgs &a, hipStream_t stream);
// True when that split kernel appends the step's token itself.
bool split_appends_itself(SplitKernel kernel);

hipError_t launch_decode_combine(const float *ws_o, const float *ws_ml, int32_t batch, int32_t num_q_heads,
                                 int32_t partials, int32_t head_dim, float *out, hipStream_t stream);

// The device address of the library's static decode workspace
// (kScratchBytes, 256-byte aligned) on the current device, looked up once
// per device; for the entry point that allocates nothing.
constexpr int64_t kScratchBytes = int64_t(32) << 20;
hipError_t scratch_for_current_device(void **out);

// Streaming read of `blocks` 9216-byte blocks (measurement utility).
hipError_t launch_read_probe(const uint8_t *buf, int64_t blocks, uint32_t *sink, hipStream_t stream);
// The configurable read probes (loads_per_lane 1, 2, 4, 8 or 16; bytes a
// multiple of 1024 * loads_per_lane).
hipError_t launch_stream_probe(const uint8_t *src, uint8_t *dst, int64_t units, int read_bytes, int write_bytes,
                               bool paired, int workgroups, uint32_t *sink, hipStream_t stream);
hipError_t launch_read_probe_config(const uint8_t *buf, int64_t bytes, int loads_per_lane, int workgroups,
                                    bool to_lds, uint32_t *sink, hipStream_t stream);

// Integer formats of the bit-width sweep (fp4kv_int.hip).
struct IntQuantArgs {
    const uint16_t *x;           // bf16 [batch][tokens][H][D]
    uint8_t *codes;              // [batch][H][tokens][D * bits / 8]
    uint16_t *scales;            // fp16: per token [batch][H][tokens], per channel [batch][H][D]
    int64_t batch, tokens;
    int32_t num_kv_heads, head_dim, bits;   // bits 2, 4, 8, or 16 (bf16 copy)
    bool per_channel;
};

struct IntDecodeArgs {
    const uint8_t *k_codes, *v_codes;
    const uint16_t *k_scales, *v_scales;
    const uint16_t *q;           // bf16 [batch][num_q_heads][D]
    int64_t tokens;
    int32_t batch, num_kv_heads, num_q_heads, group, head_dim, bits;
    int32_t splits, chunks_per_split;       // 256-token chunks per split
    bool k_per_channel, v_per_channel;
    float scale_log2e;
    float *ws_o, *ws_ml;         // partials, as for the FP4 decode
    float *out;
};

hipError_t launch_int_quantize(const IntQuantArgs &q, hipStream_t stream);
// split kernel followed by the combine kernel
hipError_t launch_int_decode(const IntDecodeArgs &a, hipStream_t stream);

}  // namespace fp4kv
