// HIP kernels for the FP4 KV cache on gfx950 (CDNA4, wave64).
//
//   quantize_append_kernel   bf16 K/V rows -> E2M1 codes + E4M3 scales at slots
//   decode_split_valu        split-K decode attention, one wave per
//                            (context split, KV head, sequence)
//   decode_combine_few       merges the splits' (max, sum, output) partials,
//                            one wave per row (up to 32 partials)
//   decode_combine           the same merge, one workgroup per row (more partials)
//
// Number formats ("Quantising the KV cache", numerics-explained, Code
// section): E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 with the sign in bit 3
// of the nibble; E4M3 (OCP FN) scales, bias 7, largest finite 448, smallest
// subnormal 2^-9.
#include <cstdint>

#include <hip/hip_runtime.h>

#include "fp4kv_internal.h"
#include "fp4kv_merge.h"
#include "fp4kv_quant.h"

namespace fp4kv {
namespace {

using namespace quant;

constexpr int kPage = 64;                 // tokens per page == lanes per wave
constexpr int64_t kRunKernelMinTokens = 512;   // appends this long use 16-token slices

// K of one token's 16-channel block: its 8 code bytes and its scale byte.
template <int D>
__device__ __forceinline__ void append_k(uint8_t *base, const CacheGeom &g, int off, int blk, const uint16_t *src)
{
    uint32_t w[8], lo, hi, sc;
    load_block16(src, w);
    quantize_block16(w, lo, hi, sc);
    *reinterpret_cast<uint2 *>(base + g.k_codes_off + off * (D / 2) + 8 * blk) = make_uint2(lo, hi);
    base[g.k_scales_off + off * (D / 16) + blk] = static_cast<uint8_t>(sc);
}

// V of one token's block, placed nibble by nibble.  A code byte is shared
// with the neighbouring token, which another thread of the same call may be
// writing, so each nibble is changed with one atomic XOR of (old ^ new) on its
// dword.  The old nibble comes from a plain load: no other thread writes this
// token's nibble, so the load sees its current value whatever happens to the
// other nibbles, and XORs on disjoint bits commute.
template <int D>
__device__ __forceinline__ void append_v_token(uint8_t *base, const CacheGeom &g, int off, int blk,
                                               const uint16_t *src)
{
    uint32_t w[8], lo, hi, sc;
    load_block16(src, w);
    quantize_block16(w, lo, hi, sc);
    const int shift = 4 * (off & 7);
    const int word = ((off & 15) >> 3) * 4;
    uint32_t *dw[16];
    uint32_t cur[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        dw[i] = reinterpret_cast<uint32_t *>(base + g.v_codes_off + v_code_row<D>(off, 16 * blk + i) + word);
        cur[i] = *dw[i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t nib = ((i < 8 ? lo : hi) >> (4 * (i & 7))) & 0xFu;
        atomicXor(dw[i], (((cur[i] >> shift) ^ nib) & 0xFu) << shift);
    }
    base[g.v_scales_off + v_scale_byte<D>(off, blk)] = static_cast<uint8_t>(sc);
}

// One token's block `blk` of KV head `head` at `slot`; slots outside the
// pool (padding, negative) are skipped.
template <int D>
__device__ __forceinline__ void append_token_fp4(const CacheGeom &g, const uint16_t *ksrc, const uint16_t *vsrc,
                                                 int64_t slot, int head, int blk, uint8_t *cache)
{
    if (slot < 0 || slot >= g.num_pages * kPage)
        return;
    uint8_t *base = cache + (slot / kPage) * g.page_stride + head * g.head_stride;
    const int off = static_cast<int>(slot % kPage);
    append_k<D>(base, g, off, blk, ksrc);
    append_v_token<D>(base, g, off, blk, vsrc);
}

// One thread per (token, KV head, 16-channel block); for small appends such
// as one token per sequence.  Consecutive threads read consecutive 32-byte
// blocks of the bf16 rows.
template <int D>
__global__ __launch_bounds__(256) void append_tokens_kernel(
    CacheGeom g, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, int64_t n_tokens,
    const int64_t *__restrict__ slots, uint8_t *__restrict__ cache)
{
    constexpr int NB = D / 16;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= n_tokens * g.num_kv_heads * NB)
        return;
    const int blk = static_cast<int>(idx % NB);
    const int64_t th = idx / NB;                        // token * H_kv + head
    const int head = static_cast<int>(th % g.num_kv_heads);
    append_token_fp4<D>(g, k + th * D + 16 * blk, v + th * D + 16 * blk, slots[th / g.num_kv_heads], head, blk,
                        cache);
}

// Transpose an 8 x 8 matrix of nibbles held as 8 dwords (dword i, nibble j
// -> dword j, nibble i): swap the off-diagonal 1x1, then 2x2, then 4x4
// nibble blocks of each 2x2 block pair.
__device__ __forceinline__ void transpose_nibbles8(uint32_t *r)
{
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const uint32_t a = r[i], b = r[i + 1];
        r[i] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
        r[i + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
    }
#pragma unroll
    for (int i = 0; i < 8; i += (i % 4 == 1) ? 3 : 1) {
        const uint32_t a = r[i], b = r[i + 2];
        r[i] = (a & 0x00FF00FFu) | ((b << 8) & 0xFF00FF00u);
        r[i + 2] = ((a >> 8) & 0x00FF00FFu) | (b & 0xFF00FF00u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a = r[i], b = r[i + 4];
        r[i] = (a & 0x0000FFFFu) | (b << 16);
        r[i + 4] = (a >> 16) | (b & 0xFFFF0000u);
    }
}

// One thread per (slice of 16 consecutive input tokens, KV head, 16-channel
// block); for prefills and other long appends.  When the slice's slots are
// 16 consecutive slots starting at a multiple of 16 -- one 16-token slice of
// a page -- the thread owns whole V code rows (16 tokens of one channel, 8
// bytes) and the slice's 16 V scale bytes of its block: its 16 channels'
// rows are 128 contiguous bytes, written with 16-byte stores, and the
// lanes of a wave (the blocks of one head) cover whole 1 KB stretches.
// Otherwise it places each token as the per-token kernel does.  k and v are
// not restrict-qualified here: with the qualifier the compiler may move their
// loads across the barriers that keep only a few rows live at a time.
template <int D>
__global__ __launch_bounds__(256) void append_slices_kernel(
    CacheGeom g, const uint16_t *k, const uint16_t *v, int64_t n_tokens,
    const int64_t *__restrict__ slots, uint8_t *__restrict__ cache)
{
    constexpr int NB = D / 16;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t n_slices = (n_tokens + 15) / 16;
    if (idx >= n_slices * g.num_kv_heads * NB)
        return;
    const int blk = static_cast<int>(idx % NB);
    const int64_t sh = idx / NB;                        // slice * H_kv + head
    const int head = static_cast<int>(sh % g.num_kv_heads);
    const int64_t t0 = (sh / g.num_kv_heads) * 16;
    const int n = static_cast<int>(n_tokens - t0 < 16 ? n_tokens - t0 : 16);
    const int64_t row_stride = static_cast<int64_t>(g.num_kv_heads) * D;   // one input token
    const uint16_t *ksrc = k + t0 * row_stride + head * D + 16 * blk;
    const uint16_t *vsrc = v + t0 * row_stride + head * D + 16 * blk;

    uint32_t w[2][4][8];                                // rows of two rounds
    auto load_round = [&](int r, uint32_t (&rows)[4][8]) {
        const uint16_t *src = (r < 4 ? ksrc : vsrc) + 4 * (r & 3) * row_stride;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            load_block16(src + i * row_stride, rows[i]);
    };
    // The slice's 16 slots with all their loads in flight at once (a loop
    // that stops at the first break issues them one at a time, each after
    // the last has arrived), and the first round of K rows beside them:
    // neither needs the other, so the check costs no round trip of its own.
    // (When the slice is not whole the rows go unused.)
    int64_t sl[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        sl[i] = i < n ? slots[t0 + i] : -1;
    if (n == 16)
        load_round(0, w[0]);
    asm volatile("" ::: "memory");
    const int64_t s0 = sl[0];
    bool whole = n == 16 && s0 >= 0 && s0 % 16 == 0 && s0 + 16 <= g.num_pages * kPage;
#pragma unroll
    for (int i = 1; i < 16; ++i)
        whole = whole & (sl[i] == s0 + i);
    if (!whole) {
        for (int i = 0; i < n; ++i)
            append_token_fp4<D>(g, ksrc + i * row_stride, vsrc + i * row_stride, slots[t0 + i], head, blk, cache);
        return;
    }
    uint8_t *base = cache + (s0 / kPage) * g.page_stride + head * g.head_stride;
    const int off0 = static_cast<int>(s0 % kPage);
    // the head's NB threads are consecutive lanes (NB divides 64), all on
    // this path together (`whole` is a property of the slice)
    const int lane_head0 = (threadIdx.x & 63) - blk;
    // Eight rounds of four tokens' rows: K of tokens 0-15 (rounds 0-3), then
    // V (rounds 4-7).  Each round's loads are issued before the previous
    // round's arithmetic, so that a wave has rows in flight while it
    // computes: a prefill's waves all fit on the GPU at once, and with one
    // round at a time they would all load, then all compute, in lockstep.
    // V: nibble rows of channels 16*blk + c, tokens off0 .. off0 + 15.  Per
    // 8 tokens the codes come out token-major (dword i = token i, nibble c =
    // channel c); an 8 x 8 nibble transpose makes them channel-major (dword
    // c = channel c, nibble i = token i), which is a V code row's half.
    uint32_t vd[2][16];                                 // [token half][channel]
    uint32_t vs[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (r + 1 < 8)
            load_round(r + 1, w[(r + 1) & 1]);
        asm volatile("" ::: "memory");
        uint32_t (&rows)[4][8] = w[r & 1];
        if (r < 4) {
            uint32_t ks = 0;                            // this block's scale codes of the round's 4 tokens
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t lo, hi, sc;
                quantize_block16(rows[i], lo, hi, sc);
                const int off = off0 + 4 * r + i;
                *reinterpret_cast<uint2 *>(base + g.k_codes_off + off * (D / 2) + 8 * blk) = make_uint2(lo, hi);
                ks |= sc << (8 * i);
            }
            // The 4 tokens' K scale rows (NB bytes each, consecutive) are
            // 4 * NB contiguous bytes: lane blk of the head stores their
            // dword blk, gathering byte m from lane (4 blk + m) % NB, the
            // block of that byte, whose codes hold it at token (4 blk + m) / NB.
            uint32_t dw = 0;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int b = 4 * blk + m;
                const uint32_t from = __shfl(ks, lane_head0 + b % NB);
                dw |= ((from >> (8 * (b / NB))) & 0xFFu) << (8 * m);
            }
            *reinterpret_cast<uint32_t *>(base + g.k_scales_off + (off0 + 4 * r) * NB + 4 * blk) = dw;
        } else {
            const int h = (r - 4) >> 1, q = (r - 4) & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t sc;
                quantize_block16(rows[i], vd[h][4 * q + i], vd[h][8 + 4 * q + i], sc);
                vs[2 * h + q] |= sc << (8 * i);
                // the codes are wanted here, not at the stores: without this
                // the compiler defers the arithmetic past later loads and
                // holds several rounds of rows at once
                asm volatile("" : "+v"(vd[h][4 * q + i]), "+v"(vd[h][8 + 4 * q + i]));
            }
            asm volatile("" : "+v"(vs[2 * h + q]));
            if (q == 1) {
                transpose_nibbles8(&vd[h][0]);
                transpose_nibbles8(&vd[h][8]);
            }
        }
        // the round after next loads into these rows: not before this arithmetic
        asm volatile("" ::: "memory");
    }
    uint4 *vrow = reinterpret_cast<uint4 *>(base + g.v_codes_off + v_code_row<D>(off0, 16 * blk));
#pragma unroll
    for (int c = 0; c < 16; c += 2)
        vrow[c / 2] = make_uint4(vd[0][c], vd[1][c], vd[0][c + 1], vd[1][c + 1]);
    *reinterpret_cast<uint4 *>(base + g.v_scales_off + v_scale_byte<D>(off0, blk)) = make_uint4(vs[0], vs[1], vs[2], vs[3]);
}

// One token's block `blk` of KV head `head` at `slot` in an FP8 cache; slots
// outside the pool are skipped.  With per-token scales the D/16 lanes of a
// (token, head) -- consecutive and aligned, and all skipped or all not --
// find the row's scale together, and the first stores it.
template <int D>
__device__ __forceinline__ void append_token_fp8(const CacheGeom &g, const uint16_t *ksrc, const uint16_t *vsrc,
                                                 int64_t slot, int head, int blk, uint8_t *cache)
{
    if (slot < 0 || slot >= g.num_pages * kPage)
        return;
    uint8_t *base = cache + (slot / kPage) * g.page_stride + head * g.head_stride;
    const int off = static_cast<int>(slot % kPage);
    uint32_t w[8];
    load_block16(ksrc, w);
    float s = g.k_scale;
    if (g.token_scales) {
        const uint32_t sc = row_scale_code_e4m3<D / 16>(w);
        s = fp16_value(sc);
        if (blk == 0)
            *reinterpret_cast<uint16_t *>(base + g.k_scales_off + 2 * off) = static_cast<uint16_t>(sc);
    }
    uint32_t kc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const uint32_t bits = (c & 1) ? (w[c >> 1] >> 16) : (w[c >> 1] & 0xFFFFu);
        kc[c >> 2] |= fp8_code(bits, s) << (8 * (c & 3));
    }
    *reinterpret_cast<uint4 *>(base + g.k_codes_off + off * D + 16 * blk) = make_uint4(kc[0], kc[1], kc[2], kc[3]);
    load_block16(vsrc, w);
    s = g.v_scale;
    if (g.token_scales) {
        const uint32_t sc = row_scale_code_e4m3<D / 16>(w);
        s = fp16_value(sc);
        if (blk == 0)
            *reinterpret_cast<uint16_t *>(base + g.v_scales_off + 2 * off) = static_cast<uint16_t>(sc);
    }
    uint8_t *vrow = base + g.v_codes_off + ((((off >> 4) * 2 + ((off >> 3) & 1)) * D + 16 * blk) * 8) + (off & 7);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const uint32_t bits = (c & 1) ? (w[c >> 1] >> 16) : (w[c >> 1] & 0xFFFFu);
        vrow[8 * c] = static_cast<uint8_t>(fp8_code(bits, s));
    }
}

// One thread per (token, KV head, 16-channel block).  K: the block's 16
// codes are one 16-byte store into the token's row.  V: channel 16*blk + i
// of the token goes to byte (off % 8) of row (slice, half, channel); every
// byte belongs to one token, so no read-modify-write is needed.
template <int D>
__global__ __launch_bounds__(256) void append_fp8_kernel(
    CacheGeom g, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, int64_t n_tokens,
    const int64_t *__restrict__ slots, uint8_t *__restrict__ cache)
{
    constexpr int NB = D / 16;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= n_tokens * g.num_kv_heads * NB)
        return;
    const int blk = static_cast<int>(idx % NB);
    const int64_t th = idx / NB;                        // token * H_kv + head
    const int head = static_cast<int>(th % g.num_kv_heads);
    append_token_fp8<D>(g, k + th * D + 16 * blk, v + th * D + 16 * blk, slots[th / g.num_kv_heads], head, blk,
                        cache);
}

// The decode step's own token, for the split kernels that do not append it
// themselves: one thread per (sequence, KV head, 16-channel block) places
// k_new / v_new of sequence b at position seq_lens[b] - 1 through the page
// table.  Empty sequences, lengths past the page table and out-of-range page
// ids are skipped.
template <int D, bool FP8>
__global__ __launch_bounds__(256) void append_last_kernel(DecodeArgs a)
{
    constexpr int NB = D / 16;
    const CacheGeom &g = a.geom;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= static_cast<int64_t>(a.batch) * g.num_kv_heads * NB)
        return;
    const int blk = static_cast<int>(idx % NB);
    const int64_t bh = idx / NB;                        // sequence * H_kv + head
    const int head = static_cast<int>(bh % g.num_kv_heads);
    const int b = static_cast<int>(bh / g.num_kv_heads);
    const int len = a.seq_lens[b];
    if (len < 1 || len > a.max_pages * kPage)            // nothing to place, or a position past the table
        return;
    const int id = a.page_table[static_cast<int64_t>(b) * a.max_pages + (len - 1) / kPage];
    const int64_t slot = (id >= 0 && id < g.num_pages) ? static_cast<int64_t>(id) * kPage + (len - 1) % kPage : -1;
    const uint16_t *ks = a.k_new + bh * D + 16 * blk;
    const uint16_t *vs = a.v_new + bh * D + 16 * blk;
    if constexpr (FP8)
        append_token_fp8<D>(g, ks, vs, slot, head, blk, a.cache_w);
    else
        append_token_fp4<D>(g, ks, vs, slot, head, blk, a.cache_w);
}

// ----------------------------------------------------------------- decode

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ float bf16_to_float(uint16_t b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Split-K decode attention on the vector ALUs.  Workgroups of four waves per
// (4 context chunks, KV head, sequence), one chunk per wave, merged in LDS at
// the end.  For each 64-token page of a wave's chunk:
//   scores: lane = token; the lane reads its K row (D/2 code bytes and D/16
//           scale bytes), converts the codes and dots them with the GM query
//           rows held in LDS (the scale is applied to each 16-channel partial
//           dot, which is the same sum regrouped);
//   softmax: running max per query head from a wave reduction, rescale factor
//           alpha = 2^(m_old - m_new), probabilities p = 2^(z - m_new) into LDS;
//   values: lane = channel pair; the lane reads its two channels' V codes
//           and its block's scales slice by slice and accumulates p * v for
//           both channels of the pair.
template <int D, int GM>
__global__ __launch_bounds__(kGroupThreads) void decode_split_valu(DecodeArgs a)
{
    constexpr int NB = D / 16;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: keeps the page loop scalar
    // grid (KV head, sequence, partial): the partial index varies slowest, so
    // the chunks nearest the start of every sequence (never empty) are
    // dispatched first, and consecutive workgroups -- which the hardware
    // deals round-robin to the XCDs -- belong to different KV heads
    const int part = blockIdx.z;
    const int sp = part * kWavesPerGroup + wave;
    const int h = blockIdx.x, b = blockIdx.y;
    const int G = a.group;

    __shared__ float q_s[GM][D];
    __shared__ float p_all[kWavesPerGroup][GM][kPage];
    __shared__ __attribute__((aligned(16))) uint8_t areas[kWavesPerGroup * merge_area_bytes<D>()];
    float (*p_s)[kPage] = p_all[wave];

    for (int i = threadIdx.x; i < GM * D; i += kGroupThreads) {
        const int gq = i / D, c = i % D;
        q_s[gq][c] = gq < G ? bf16_to_float(a.q[(static_cast<int64_t>(b) * a.num_q_heads + h * G + gq) * D + c])
                            : 0.0f;
    }
    __syncthreads();

    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_pages * kPage ? a.max_pages * kPage : len);
    const int n_pages = (len + kPage - 1) / kPage;
    const int p0 = chunk_first_page(a, sp);
    const int p1 = min(p0 + chunk_pages(a, sp), n_pages);

    float m[GM], l[GM], o0[GM], o1[GM];
#pragma unroll
    for (int gq = 0; gq < GM; ++gq) {
        m[gq] = -INFINITY; l[gq] = 0.0f; o0[gq] = 0.0f; o1[gq] = 0.0f;
    }

    const CacheGeom &g = a.geom;
    for (int pg = p0; pg < p1; ++pg) {
        const int pid = a.page_table[static_cast<int64_t>(b) * a.max_pages + pg];
        if (pid < 0 || pid >= g.num_pages)
            continue;                                   // not a page of this pool: skipped
        const uint8_t *blk = a.cache + static_cast<int64_t>(pid) * g.page_stride + h * g.head_stride;
        const int valid = min(kPage, len - pg * kPage);

        // ---- scores, lane = token
        float z[GM];
#pragma unroll
        for (int gq = 0; gq < GM; ++gq)
            z[gq] = 0.0f;
        {
            // one 16-channel block at a time, re-reading the query rows from LDS
            const uint2 *krow = reinterpret_cast<const uint2 *>(blk + g.k_codes_off + lane * (D / 2));
            const uint8_t *ksc = blk + g.k_scales_off + lane * NB;
#pragma unroll 1
            for (int nb = 0; nb < NB; ++nb) {
                const uint2 cw = krow[nb];
                const float s = e4m3_value(ksc[nb]);
                float part[GM];
#pragma unroll
                for (int gq = 0; gq < GM; ++gq)
                    part[gq] = 0.0f;
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const uint32_t word = (c < 8) ? cw.x : cw.y;
                    const float kv = e2m1_value(word >> (4 * (c & 7)));
#pragma unroll
                    for (int gq = 0; gq < GM; ++gq)
                        part[gq] = fmaf(q_s[gq][16 * nb + c], kv, part[gq]);
                }
#pragma unroll
                for (int gq = 0; gq < GM; ++gq)
                    z[gq] = fmaf(s, part[gq], z[gq]);
            }
        }
        const bool live = lane < valid;

        // ---- online softmax (base 2)
#pragma unroll
        for (int gq = 0; gq < GM; ++gq) {
            const float zz = live ? z[gq] * a.scale_log2e : -INFINITY;
            const float mx = wave_max(zz);               // finite: lane 0 is live
            const float mn = fmaxf(m[gq], mx);
            const float alpha = exp2f(m[gq] - mn);       // 0 on the first page
            const float p = live ? exp2f(zz - mn) : 0.0f;
            l[gq] = fmaf(l[gq], alpha, p);
            o0[gq] *= alpha;
            o1[gq] *= alpha;
            m[gq] = mn;
            p_s[gq][lane] = p;
        }
        // the wave's own LDS writes, in order, before its reads below
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- values, lane = channel pair (D/2 lanes), one 16-token slice at a
        //      time: channel 2*lane's 8 code bytes then channel 2*lane + 1's,
        //      two tokens per byte, and the 16 scales of the pair's block
        if (lane < D / 2) {
#pragma unroll 1
            for (int ch = 0; ch < kPage / 16; ++ch) {
                if (16 * ch >= valid)
                    break;
                const uint4 vc = *reinterpret_cast<const uint4 *>(blk + g.v_codes_off + (ch * D + 2 * lane) * 8);
                const uint4 vs = *reinterpret_cast<const uint4 *>(blk + g.v_scales_off + (ch * NB + (lane >> 3)) * 16);
                const uint32_t ce[2] = {vc.x, vc.y}, co[2] = {vc.z, vc.w};
                const uint32_t sw[4] = {vs.x, vs.y, vs.z, vs.w};
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float s = e4m3_value((sw[i >> 2] >> (8 * (i & 3))) & 0xFFu);
                    const float ve = e2m1_value(ce[i >> 3] >> (4 * (i & 7))) * s;
                    const float vo = e2m1_value(co[i >> 3] >> (4 * (i & 7))) * s;
#pragma unroll
                    for (int gq = 0; gq < GM; ++gq) {
                        const float p = p_s[gq][16 * ch + i];
                        o0[gq] = fmaf(p, ve, o0[gq]);
                        o1[gq] = fmaf(p, vo, o1[gq]);
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- this wave's state into its merge area, then one partial per workgroup
    auto area = [&](int w) { return MergeArea<D>(areas + w * merge_area_bytes<D>()); };
    const MergeArea<D> ar = area(wave);
#pragma unroll
    for (int gq = 0; gq < GM; ++gq) {
        const float lt = wave_sum(l[gq]);
        if (gq >= G)
            continue;
        if (lane == 0) {
            ar.ml[2 * gq] = m[gq];
            ar.ml[2 * gq + 1] = lt;
        }
        if (lane < D / 2)
            *reinterpret_cast<float2 *>(ar.row(gq) + 2 * lane) = make_float2(o0[gq], o1[gq]);
    }
    merge_waves_and_store<D>(area, a, b, h, part);
}

// Merge the partials of one (sequence, query head): M = max_j m_j,
// L = sum_j l_j 2^(m_j - M), out = sum_j o_j 2^(m_j - M) / L.  Partials with
// no tokens carry m = -inf and l = 0 and are skipped (their outputs are not
// read into the sums); a row with no tokens at all is written as zeros.  One
// workgroup per row (rows with many partials are few: a small batch over a
// long context).  Wave w takes every fourth batch of 16 partials, issues all
// of a batch's loads -- the (m, l) pairs and lane c's D/64 channels of each
// output -- before using any, and folds the batch into a running (M_w, L_w,
// O_w) relative to its own maximum, so the row costs one memory round trip
// per batch instead of a first pass for M; the four waves' states are then
// merged once in LDS: out = sum_w O_w 2^(M_w - M) / sum_w L_w 2^(M_w - M).
template <int D>
__global__ __launch_bounds__(256) void decode_combine(const float *__restrict__ ws_o,
                                                      const float *__restrict__ ws_ml, int num_q_heads,
                                                      int partials, float *__restrict__ out)
{
    constexpr int CL = D / 64;                          // consecutive channels per lane
    constexpr int NBT = 16;                             // partials a wave loads together
    __shared__ float part[4][D + 2];                    // per wave: O_w, then L_w and M_w
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = blockIdx.x;                     // b * num_q_heads + query head
    const int64_t b = row / num_q_heads, hq = row % num_q_heads;
    // partial j of this row: index (b * partials + j) * num_q_heads + hq
    const int64_t first = b * partials * num_q_heads + hq;
    const float2 *ml = reinterpret_cast<const float2 *>(ws_ml) + first;
    const float *o = ws_o + first * D + lane * CL;
    const int64_t stride = static_cast<int64_t>(num_q_heads) * D;

    float Mw = -INFINITY, Lw = 0.0f, O[CL];
#pragma unroll
    for (int i = 0; i < CL; ++i)
        O[i] = 0.0f;
    for (int j0 = wave * NBT; j0 < partials; j0 += 4 * NBT) {
        const int n = min(NBT, partials - j0);
        float2 mj[NBT];
        float x[NBT][CL];
        // the outputs' loads, then lane i < 16 loads pair i: one vector load
        // for the batch's pairs, issued last, so that waiting for it (the
        // counter is in order) waits for the whole batch, one round trip; as
        // 16 scalar loads the pairs went out ahead of the outputs with a wait
        // between.  Every lane then takes the 16 pairs with readlane.
#pragma unroll
        for (int i = 0; i < NBT; ++i) {
            const int64_t jj = j0 + (i < n ? i : n - 1);     // past the last: re-read it, weight zero below
#pragma unroll
            for (int c = 0; c < CL; ++c)
                x[i][c] = o[jj * stride + c];
        }
        const int li = lane < n ? lane : n - 1;
        const float2 my = ml[static_cast<int64_t>(j0 + (li < NBT ? li : NBT - 1)) * num_q_heads];
        // the scheduler would otherwise hoist the pair load and its readlanes
        // above most of the output loads (one more round trip)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NBT; ++i) {
            mj[i].x = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my.x), i));
            mj[i].y = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my.y), i));
        }
        float mb = -INFINITY;
#pragma unroll
        for (int i = 0; i < NBT; ++i)
            mb = i < n ? fmaxf(mb, mj[i].x) : mb;
        // no branch on an empty batch (it would let the compiler sink the
        // output loads below a wait for the pairs): with Mn = -inf every
        // weight below is 0 and the state stays as it is
        const float Mn = fmaxf(Mw, mb);
        const float alpha = Mw == -INFINITY ? 0.0f : exp2f(Mw - Mn);
        Lw *= alpha;
#pragma unroll
        for (int c = 0; c < CL; ++c)
            O[c] *= alpha;
#pragma unroll
        for (int i = 0; i < NBT; ++i) {
            const float w = (i < n && mj[i].x != -INFINITY) ? exp2f(mj[i].x - Mn) : 0.0f;
            Lw = fmaf(mj[i].y, w, Lw);
            // an empty partial's outputs are not meaningful (not written):
            // a zero weight leaves the sums as they are
#pragma unroll
            for (int c = 0; c < CL; ++c)
                O[c] = w != 0.0f ? fmaf(x[i][c], w, O[c]) : O[c];
        }
        Mw = Mn;
    }
#pragma unroll
    for (int c = 0; c < CL; ++c)
        part[wave][lane * CL + c] = O[c];
    if (lane == 0) {
        part[wave][D] = Lw;
        part[wave][D + 1] = Mw;
    }
    __syncthreads();
    if (wave == 0) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            M = fmaxf(M, part[w][D + 1]);
        float sc[4], Lt = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            sc[w] = part[w][D + 1] == -INFINITY ? 0.0f : exp2f(part[w][D + 1] - M);
            Lt = fmaf(part[w][D], sc[w], Lt);
        }
        const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
#pragma unroll
        for (int i = 0; i < CL; ++i) {
            const int c = lane * CL + i;
            float acc = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                acc = sc[w] != 0.0f ? fmaf(part[w][c], sc[w], acc) : acc;
            out[row * D + c] = acc * inv;
        }
    }
}

// The same merge for rows with at most PM partials: one wave per row, four
// rows per workgroup, lane l covering channels CL*l .. CL*l + CL - 1.  Every
// load of the row is issued before any result is used (partials past the
// last re-read the last one and get weight zero), and the (m, l) pairs are
// the same for the whole wave, so the merge needs no LDS and no barrier.
template <int D, int PM>
__global__ __launch_bounds__(256) void decode_combine_few(const float *__restrict__ ws_o,
                                                          const float *__restrict__ ws_ml, int64_t rows,
                                                          int num_q_heads, int partials, float *__restrict__ out)
{
    constexpr int CL = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int64_t b = row / num_q_heads, hq = row % num_q_heads;
    // partial j of this row: index (b * partials + j) * num_q_heads + hq
    const int64_t first = b * partials * num_q_heads + hq;
    const float2 *ml = reinterpret_cast<const float2 *>(ws_ml) + first;
    const float *o = ws_o + first * D + lane * CL;
    const int64_t stride = static_cast<int64_t>(num_q_heads) * D;
    float2 mj[PM];
    float x[PM][CL];
#pragma unroll
    for (int j = 0; j < PM; ++j) {
        const int jc = j < partials ? j : partials - 1;
        mj[j] = ml[static_cast<int64_t>(jc) * num_q_heads];
        if constexpr (CL == 2) {
            const float2 v = *reinterpret_cast<const float2 *>(o + jc * stride);
            x[j][0] = v.x;
            x[j][1] = v.y;
        } else {
            x[j][0] = o[jc * stride];
        }
    }
    // keep the scheduler from placing the maximum (which needs the (m, l)
    // loads) before the channel loads are issued
    __builtin_amdgcn_sched_barrier(0);
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < PM; ++j)
        M = j < partials ? fmaxf(M, mj[j].x) : M;
    float L = 0.0f, O[CL];
#pragma unroll
    for (int i = 0; i < CL; ++i)
        O[i] = 0.0f;
    // no branch on M: every weight is zero when all partials are empty
#pragma unroll
    for (int j = 0; j < PM; ++j) {
        const float w = (j < partials && mj[j].x != -INFINITY) ? exp2f(mj[j].x - M) : 0.0f;
        L = fmaf(mj[j].y, w, L);
        // an empty partial's outputs are not meaningful (not written): a
        // zero weight leaves the sums as they are
#pragma unroll
        for (int i = 0; i < CL; ++i)
            O[i] = w != 0.0f ? fmaf(x[j][i], w, O[i]) : O[i];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if constexpr (CL == 2) {
        *reinterpret_cast<float2 *>(out + row * D + lane * CL) = make_float2(O[0] * inv, O[1] * inv);
    } else {
        out[row * D + lane] = O[0] * inv;
    }
}

// Each wave reads one 9216-byte block per iteration: nine 1 KB rows, lane l
// taking bytes 16l .. 16l+15 of each, all nine loads in flight together.
__global__ __launch_bounds__(256) void read_probe(const uint8_t *__restrict__ buf, int64_t blocks,
                                                  uint32_t *sink)
{
    constexpr int64_t kBlock = 9216;
    const int lane = threadIdx.x & 63;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
    uint32_t acc = 0;
    for (int64_t b = wave; b < blocks; b += stride) {
        const uint4 *p = reinterpret_cast<const uint4 *>(buf + b * kBlock) + lane;
        uint4 x[9];
#pragma unroll
        for (int k = 0; k < 9; ++k)
            x[k] = p[64 * k];
#pragma unroll
        for (int k = 0; k < 9; ++k)
            acc ^= x[k].x ^ x[k].y ^ x[k].z ^ x[k].w;
    }
    if (acc == 0x9E3779B9u)
        sink[0] = acc;
}

// Read ceiling probes: every wave reads whole 64 * 16 * L byte stretches of
// the buffer (L 16-byte non-temporal loads per lane, all in flight together)
// in a grid-stride loop, into registers (XOR-reduced so that nothing is
// optimised away) or, as the decode kernel's page copies do, straight into
// LDS.  The buffer is read once.
template <int L>
__global__ __launch_bounds__(256) void read_probe_regs(const uint8_t *__restrict__ buf, int64_t stretches,
                                                        uint32_t *sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t waves = static_cast<int64_t>(gridDim.x) * 4;
    uint32_t acc = 0;
    for (int64_t s = wave; s < stretches; s += waves) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 *p = reinterpret_cast<const u32x4 *>(buf + s * (1024 * L)) + lane;
        u32x4 x[L];
#pragma unroll
        for (int k = 0; k < L; ++k)
            x[k] = __builtin_nontemporal_load(p + 64 * k);
#pragma unroll
        for (int k = 0; k < L; ++k)
            acc ^= x[k].x ^ x[k].y ^ x[k].z ^ x[k].w;
    }
    if (acc == 0x9E3779B9u)
        sink[0] = acc;
}

// 16 bytes per lane from global memory straight into LDS, non-temporal.
__device__ __forceinline__ void copy16_to_lds(const uint8_t *src, uint8_t *dst)
{
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 2);
}

template <int L>
__global__ __launch_bounds__(256) void read_probe_lds(const uint8_t *__restrict__ buf, int64_t stretches,
                                                       uint32_t *sink)
{
    __shared__ __attribute__((aligned(16))) uint8_t slot[4][1024 * L];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + w;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * 4;
    uint32_t acc = 0;
    for (int64_t s = wave; s < stretches; s += waves) {
        const uint8_t *p = buf + s * (1024 * L) + lane * 16;
#pragma unroll
        for (int k = 0; k < L; ++k)
            copy16_to_lds(p + 1024 * k, &slot[w][1024 * k]);
        __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0): the stretch is in LDS
        acc ^= *reinterpret_cast<const uint32_t *>(&slot[w][1024 * (lane % L) + 16 * (lane / L)]);
        __builtin_amdgcn_s_waitcnt(0xC07F);              // the read is done before the next copies
    }
    if (acc == 0x9E3779B9u)
        sink[0] = acc;
}

template <int L>
hipError_t probe_launch_l(const uint8_t *buf, int64_t stretches, dim3 grid, bool to_lds, uint32_t *sink,
                          hipStream_t stream)
{
    if (to_lds)
        read_probe_lds<L><<<grid, 256, 0, stream>>>(buf, stretches, sink);
    else
        read_probe_regs<L><<<grid, 256, 0, stream>>>(buf, stretches, sink);
    return hipGetLastError();
}

hipError_t probe_launch(const uint8_t *buf, int64_t stretches, int loads_per_lane, dim3 grid, bool to_lds,
                        uint32_t *sink, hipStream_t stream)
{
    switch (loads_per_lane) {
    case 1: return probe_launch_l<1>(buf, stretches, grid, to_lds, sink, stream);
    case 2: return probe_launch_l<2>(buf, stretches, grid, to_lds, sink, stream);
    case 4: return probe_launch_l<4>(buf, stretches, grid, to_lds, sink, stream);
    case 8: return probe_launch_l<8>(buf, stretches, grid, to_lds, sink, stream);
    case 16: return probe_launch_l<16>(buf, stretches, grid, to_lds, sink, stream);
    default: return hipErrorInvalidValue;
    }
}

// Streaming read + write probe: wave u of a grid-stride loop over units
// reads read_bytes contiguous bytes of unit u (8 loads of 16 bytes per lane
// in flight) and then writes write_bytes contiguous bytes.  PAIRED reads as
// the quantiser does: lane l takes bytes [32 l, 32 l + 32) of each 2 KB row
// in two 16-byte loads (4 rows in flight); otherwise each load instruction
// takes a whole kilobyte (lane l bytes [16 l, 16 l + 16)).
template <bool PAIRED>
__global__ __launch_bounds__(256) void stream_probe(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                    int64_t units, int read_bytes, int write_bytes, uint32_t *sink)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t waves = static_cast<int64_t>(gridDim.x) * 4;
    uint32_t acc = 0;
    for (int64_t u = wave; u < units; u += waves) {
        const uint8_t *unit = src + u * read_bytes;
        for (int at = 0; at < read_bytes; at += 8192) {      // 8 KB a step: 128 bytes per lane
            u32x4 x[8];
            if (PAIRED) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const u32x4 *p = reinterpret_cast<const u32x4 *>(unit + at + 2048 * r + 32 * lane);
                    x[2 * r] = __builtin_nontemporal_load(p);
                    x[2 * r + 1] = __builtin_nontemporal_load(p + 1);
                }
            } else {
                const u32x4 *p = reinterpret_cast<const u32x4 *>(unit + at) + lane;
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    x[k] = __builtin_nontemporal_load(p + 64 * k);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                acc ^= x[k].x ^ x[k].y ^ x[k].z ^ x[k].w;
        }
        u32x4 *q = reinterpret_cast<u32x4 *>(dst + u * write_bytes) + lane;
        for (int k = 0; k < write_bytes / 1024; ++k)
            q[64 * k] = u32x4{acc, acc + 1u, acc + 2u, acc + 3u};
    }
    if (acc == 0x9E3779B9u)
        sink[0] = acc;
}

template <int D, int GM>
hipError_t launch_split_t(const DecodeArgs &a, hipStream_t stream)
{
    const dim3 grid(a.geom.num_kv_heads, a.batch, a.partials);
    decode_split_valu<D, GM><<<grid, kGroupThreads, 0, stream>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const DecodeArgs &a, hipStream_t stream)
{
    if (a.group <= 1) return launch_split_t<D, 1>(a, stream);
    if (a.group <= 2) return launch_split_t<D, 2>(a, stream);
    if (a.group <= 4) return launch_split_t<D, 4>(a, stream);
    if (a.group <= 8) return launch_split_t<D, 8>(a, stream);
    return launch_split_t<D, 16>(a, stream);
}

}  // namespace

hipError_t launch_quantize_append(const CacheGeom &g, const uint16_t *k, const uint16_t *v,
                                  int64_t n_tokens, const int64_t *slots, uint8_t *cache,
                                  hipStream_t stream)
{
    const int64_t per_token = static_cast<int64_t>(g.num_kv_heads) * (g.head_dim / 16);
    if (g.fp8) {
        const int64_t blocks = (n_tokens * per_token + 255) / 256;
        if (g.head_dim == 64)
            append_fp8_kernel<64><<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(g, k, v, n_tokens, slots, cache);
        else
            append_fp8_kernel<128><<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(g, k, v, n_tokens, slots, cache);
    } else if (n_tokens >= kRunKernelMinTokens) {
        const int64_t blocks = ((n_tokens + 15) / 16 * per_token + 255) / 256;
        if (g.head_dim == 64)
            append_slices_kernel<64><<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(g, k, v, n_tokens, slots, cache);
        else
            append_slices_kernel<128><<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(g, k, v, n_tokens, slots, cache);
    } else {
        const int64_t blocks = (n_tokens * per_token + 255) / 256;
        if (g.head_dim == 64)
            append_tokens_kernel<64><<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(g, k, v, n_tokens, slots, cache);
        else
            append_tokens_kernel<128><<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(g, k, v, n_tokens, slots, cache);
    }
    return hipGetLastError();
}

hipError_t launch_split_valu(const DecodeArgs &a, hipStream_t stream)
{
    return a.geom.head_dim == 64 ? launch_split_d<64>(a, stream) : launch_split_d<128>(a, stream);
}

hipError_t launch_append_last(const DecodeArgs &a, hipStream_t stream)
{
    const int64_t threads = static_cast<int64_t>(a.batch) * a.geom.num_kv_heads * (a.geom.head_dim / 16);
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
    if (a.geom.fp8 && a.geom.head_dim == 64)
        append_last_kernel<64, true><<<grid, 256, 0, stream>>>(a);
    else if (a.geom.fp8)
        append_last_kernel<128, true><<<grid, 256, 0, stream>>>(a);
    else if (a.geom.head_dim == 64)
        append_last_kernel<64, false><<<grid, 256, 0, stream>>>(a);
    else
        append_last_kernel<128, false><<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
}

bool split_appends_itself(SplitKernel kernel)
{
    return kernel == SplitKernel::fp8 || kernel == SplitKernel::mfma_staged;
}

hipError_t launch_decode_split(const DecodeArgs &a, SplitKernel kernel, hipStream_t stream)
{
    DecodeArgs m = a;
    if (a.k_new && !split_appends_itself(kernel)) {
        const hipError_t e = launch_append_last(a, stream);
        if (e != hipSuccess)
            return e;
        m.k_new = m.v_new = nullptr;
        m.cache_w = nullptr;
    }
    switch (kernel) {
    case SplitKernel::fp8:
        return launch_split_fp8(m, stream);
    case SplitKernel::valu:
        return launch_split_valu(m, stream);
    case SplitKernel::mfma_direct:
        m.staged = false;
        return launch_split_mfma(m, stream);
    case SplitKernel::mfma_staged:
        m.staged = true;
        return launch_split_mfma(m, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const float *ws_o, const float *ws_ml, int32_t batch, int32_t num_q_heads,
                                 int32_t partials, int32_t head_dim, float *out, hipStream_t stream)
{
    const int64_t rows = static_cast<int64_t>(batch) * num_q_heads;
    if (partials <= 32) {
        // one wave per row, four rows per workgroup
        const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
        if (head_dim == 64) {
            if (partials <= 16)
                decode_combine_few<64, 16><<<grid, 256, 0, stream>>>(ws_o, ws_ml, rows, num_q_heads, partials, out);
            else
                decode_combine_few<64, 32><<<grid, 256, 0, stream>>>(ws_o, ws_ml, rows, num_q_heads, partials, out);
        } else {
            if (partials <= 16)
                decode_combine_few<128, 16><<<grid, 256, 0, stream>>>(ws_o, ws_ml, rows, num_q_heads, partials, out);
            else
                decode_combine_few<128, 32><<<grid, 256, 0, stream>>>(ws_o, ws_ml, rows, num_q_heads, partials, out);
        }
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>(rows));   // one workgroup per row
    if (head_dim == 64)
        decode_combine<64><<<grid, 256, 0, stream>>>(ws_o, ws_ml, num_q_heads, partials, out);
    else
        decode_combine<128><<<grid, 256, 0, stream>>>(ws_o, ws_ml, num_q_heads, partials, out);
    return hipGetLastError();
}

hipError_t launch_read_probe_config(const uint8_t *buf, int64_t bytes, int loads_per_lane, int workgroups,
                                    bool to_lds, uint32_t *sink, hipStream_t stream)
{
    return probe_launch(buf, bytes / (1024 * loads_per_lane), loads_per_lane, dim3(static_cast<unsigned>(workgroups)),
                        to_lds, sink, stream);
}

hipError_t launch_stream_probe(const uint8_t *src, uint8_t *dst, int64_t units, int read_bytes, int write_bytes,
                               bool paired, int workgroups, uint32_t *sink, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(workgroups));
    if (paired)
        stream_probe<true><<<grid, 256, 0, stream>>>(src, dst, units, read_bytes, write_bytes, sink);
    else
        stream_probe<false><<<grid, 256, 0, stream>>>(src, dst, units, read_bytes, write_bytes, sink);
    return hipGetLastError();
}

hipError_t launch_read_probe(const uint8_t *buf, int64_t blocks, uint32_t *sink, hipStream_t stream)
{
    const int64_t groups = (blocks + 3) / 4;
    const dim3 grid(static_cast<unsigned>(groups < 8192 ? groups : 8192));
    read_probe<<<grid, 256, 0, stream>>>(buf, blocks, sink);
    return hipGetLastError();
}

}  // namespace fp4kv
