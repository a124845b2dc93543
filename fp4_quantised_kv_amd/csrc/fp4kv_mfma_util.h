// Matrix-core decode pieces shared by the FP4 and FP8 kernels: operand
// types and conversions, the lane-swap max, the online softmax over score
// tiles, the query operand, the per-wave state and its merge-area image, and
// the page range of a wave's chunk.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "fp4kv_internal.h"
#include "fp4kv_merge.h"
#include "fp4kv_quant.h"

namespace fp4kv {
namespace mfma {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));

constexpr int kPage = 64;
constexpr float kRescaleSlack = 8.0f;      // base-2 headroom before the reference max moves

template <int SEL>
__device__ __forceinline__ half2_t fp4x2(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

template <bool HI>
__device__ __forceinline__ half2_t fp8x2(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

__device__ __forceinline__ half8_t cat(half2_t a, half2_t b, half2_t c, half2_t d)
{
    const half4_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const half4_t cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ half2_t pk_rtz(float a, float b)
{
    return __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// Max over the four lanes l, l^16, l^32, l^48 (one query column of a C
// tile), with the gfx950 lane-swap instructions instead of LDS shuffles.
__device__ __forceinline__ float xor_max(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Keep the bytes of a dword whose token index (t0 + byte) is below `valid`.
__device__ __forceinline__ uint32_t keep_valid_bytes(uint32_t w, int t0, int valid)
{
    const int n = valid - t0;
    if (n >= 4)
        return w;
    if (n <= 0)
        return 0u;
    return w & ((1u << (8 * n)) - 1u);
}

// Running state of one wave over its chunk.
template <int D>
struct SplitState {
    float m_ref;
    float4_t acc[D / 16];                 // O^T tiles: (pair block u, parity) -> index 2u + parity
    float4_t lacc;
};

// Page-local token of score tile t, row `row`.
__device__ __forceinline__ int tile_token(int t, int row) { return 16 * (row >> 2) + 4 * t + (row & 3); }

// Online softmax over NT score tiles (NT = 2: one 32-token half page; 4: a
// whole page), with a lazily moved reference max; leaves the probabilities
// as the value product's B operands, hi and lo fp16 parts per tile pair.
// z holds unscaled scores, already -inf for tokens past the valid length.
template <int D, int NT>
__device__ __forceinline__ void softmax_tiles(const float (&z)[NT][4], SplitState<D> &st, float zscale,
                                              half8_t (&pf)[NT / 2], half8_t (&pl)[NT / 2])
{
    const half8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};
    float mx = z[0][0];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            mx = fmaxf(mx, z[t][e]);
    mx = xor_max(mx) * zscale;                          // zscale > 0: max commutes with it
    const bool move = mx > st.m_ref + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float m_new = move ? mx : st.m_ref;
        const float alpha = move ? __builtin_amdgcn_exp2f(st.m_ref - m_new) : 1.0f;
        st.m_ref = m_new;
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
            st.acc[t] *= alpha;
        st.lacc *= alpha;
    }
    // p = hi + lo with both parts in fp16 (hi truncated, lo the truncated
    // remainder): the value and denominator products see p to ~2^-21
    // relative, so fp16 operands cost no accuracy against fp32.
    // -1 held in a register the compiler cannot see through, so that
    // p - float(hi) stays one mixed-precision FMA instead of a conversion
    // and a subtraction
    float minus_one = -1.0f;
    asm volatile("" : "+s"(minus_one));
    // a column that has seen no token yet (possible with several query
    // tokens: its causal limit can lie before this page) keeps m = -inf and
    // must get p = 0, not exp2(-inf + inf)
    const float m_sub = st.m_ref == -INFINITY ? 0.0f : st.m_ref;
#pragma unroll
    for (int kt = 0; kt < NT / 2; ++kt) {
        float p[8], q[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[2 * kt][e], zscale, -m_sub));
            p[4 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[2 * kt + 1][e], zscale, -m_sub));
        }
        pf[kt] = cat(pk_rtz(p[0], p[1]), pk_rtz(p[2], p[3]), pk_rtz(p[4], p[5]), pk_rtz(p[6], p[7]));
#pragma unroll
        for (int e = 0; e < 8; ++e)
            q[e] = __builtin_fmaf(static_cast<float>(pf[kt][e]), minus_one, p[e]);
        pl[kt] = cat(pk_rtz(q[0], q[1]), pk_rtz(q[2], q[3]), pk_rtz(q[4], q[5]), pk_rtz(q[6], q[7]));
        st.lacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[kt], st.lacc, 0, 0, 0);
        st.lacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pl[kt], st.lacc, 0, 0, 0);
    }
}

// Cache policy of the copies: non-temporal.  The cache is read once per
// step; without the hint the stream evicts the partial results this kernel
// writes from L2, and their write-back to HBM interleaved with the stream
// costs about 10 % of the kernel's time (measured at 32 x 32K context).
constexpr int kStream = 2;                // the NT bit of the instruction's cache-policy field

// gfx9 s_waitcnt immediates (expcnt and lgkmcnt left free): at most n vector
// memory operations outstanding; and all LDS accesses done.
template <int N>
__device__ __forceinline__ void wait_vmem_at_most()
{
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
constexpr int kWaitLds = 0xC07F;

// ---- query operand, per-wave state, chunk geometry

// Query columns: column col is query token col / G, head h*G + col % G of
// the group (q_tokens * G <= 16 columns; one query token: column = head).
__device__ __forceinline__ int query_columns(const DecodeArgs &a) { return (a.q_tokens > 1 ? a.q_tokens : 1) * a.group; }

// Tokens a column may not see at the end of the context: query token i of
// q_tokens sees the first len - (q_tokens - 1 - i) tokens (causal).
__device__ __forceinline__ int column_shortfall(const DecodeArgs &a, int col)
{
    return col < query_columns(a) ? (a.q_tokens > 1 ? a.q_tokens : 1) - 1 - col / a.group : 0;
}

// Query rows of (sequence b, KV head h) as bf16 bits: lane (col, jj) holds
// channels jj*D/4 .. +D/4 of query column col; columns past the last load a
// valid row and are zeroed after the load (no divergent loads).
template <int D>
__device__ __forceinline__ void load_q_bits(const DecodeArgs &a, int b, int h, int col, int jj,
                                            uint32_t (&qbits)[D / 8])
{
    constexpr int CPL = D / 4;
    const int G = a.group;
    const int S = a.q_tokens > 1 ? a.q_tokens : 1;
    const bool live = col < S * G;
    const int c = live ? col : 0;
    const int64_t row = (static_cast<int64_t>(b) * S + c / G) * a.num_q_heads + h * G + c % G;
    const uint16_t *qrow = a.q + row * D + jj * CPL;
#pragma unroll
    for (int i = 0; i < CPL / 8; ++i) {
        const uint4 x = reinterpret_cast<const uint4 *>(qrow)[i];
        qbits[4 * i] = x.x; qbits[4 * i + 1] = x.y; qbits[4 * i + 2] = x.z; qbits[4 * i + 3] = x.w;
    }
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i)
        qbits[i] = live ? qbits[i] : 0u;
}

// The B operand of the score product: q times 2^kq, kq putting the wave's
// largest |q| in [2^14, 2^15) (exact for bf16 inputs), in fp16; zscale
// undoes 2^kq and applies softmax_scale * log2(e).  Every lane of the wave
// must take part (wave-wide maximum).
template <int D>
__device__ __forceinline__ void make_q_operand(const uint32_t (&qbits)[D / 8], float scale_log2e,
                                               half8_t (&qf)[D / 32], float &zscale)
{
    float qmax = 0.0f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
        qmax = fmaxf(qmax, __uint_as_float((qbits[i] & 0x7FFFu) << 16));
        qmax = fmaxf(qmax, __uint_as_float(qbits[i] & 0x7FFF0000u));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        qmax = fmaxf(qmax, __shfl_xor(qmax, o));
    int kq = 0;
    if (qmax > 0.0f)
        kq = 14 - (static_cast<int>((__float_as_uint(qmax) >> 23) & 0xFF) - 127);
    kq = kq > 100 ? 100 : kq;
    const float qscale = __builtin_ldexpf(1.0f, kq);
    zscale = scale_log2e * __builtin_ldexpf(1.0f, -kq);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = qbits[4 * i + e];
            qf[i][2 * e] = static_cast<_Float16>(__uint_as_float(w << 16) * qscale);
            qf[i][2 * e + 1] = static_cast<_Float16>(__uint_as_float(w & 0xFFFF0000u) * qscale);
        }
    }
}

template <int D>
__device__ __forceinline__ void init_state(SplitState<D> &st)
{
    st.m_ref = -INFINITY;
    st.lacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
        st.acc[t] = st.lacc;
}

// A wave's state into its merge area: lane (col = query column, jj) holds
// channels 2*(16u + 4jj + r) + parity, i.e. 32u + 8jj + 0..7.
template <int D>
__device__ __forceinline__ void state_to_area(const MergeArea<D> &ar, const SplitState<D> &st, int col, int jj,
                                              int columns)
{
    if (col < columns) {
        float *o = ar.row(col);
#pragma unroll
        for (int u = 0; u < D / 32; ++u) {
            const int c0 = 32 * u + 8 * jj;
            *reinterpret_cast<float4 *>(o + c0) =
                make_float4(st.acc[2 * u][0], st.acc[2 * u + 1][0], st.acc[2 * u][1], st.acc[2 * u + 1][1]);
            *reinterpret_cast<float4 *>(o + c0 + 4) =
                make_float4(st.acc[2 * u][2], st.acc[2 * u + 1][2], st.acc[2 * u][3], st.acc[2 * u + 1][3]);
        }
        if (jj == 0) {
            ar.ml[2 * col] = st.m_ref;
            ar.ml[2 * col + 1] = st.lacc[0];
        }
    }
}

// Page range of a wave's chunk and its first 64 page ids.  The ids are
// bounded by the table, not by the length, so their load need not wait for
// the length.
struct Chunk {
    int h, b, part;
    int p0, p1, len;
    const int32_t *ptab;
};

// The part of a wave's chunk that needs no memory read: its unshifted first
// page and page count.  The page ids load from here.
__device__ __forceinline__ Chunk chunk_start(const DecodeArgs &a, int h, int b, int part, int wave)
{
    Chunk c;
    c.h = h; c.b = b; c.part = part;
    c.ptab = a.page_table + static_cast<int64_t>(b) * a.max_pages;
    const int k = part * kWavesPerGroup + wave;
    c.p0 = chunk_first_page(a, k);
    c.p1 = c.p0 + chunk_pages(a, k);
    c.len = 0;
    return c;
}

// The part that needs the context length: the length itself, the window's
// shift of the start and the end clamped to the context.  Kernels read it
// after issuing the loads that do not need it, so that its load overlaps
// theirs instead of preceding them.
__device__ __forceinline__ void chunk_clamp(const DecodeArgs &a, Chunk &c)
{
    int len = a.seq_lens[c.b];
    len = len < 0 ? 0 : (len > a.max_pages * kPage ? a.max_pages * kPage : len);
    c.len = len;
    const int pages = c.p1 - c.p0;
    if (a.window > 0) {
        // chunks start at the page of the earliest token any query column
        // sees: the first query token's prefix end minus the window
        const int first = len - ((a.q_tokens > 1 ? a.q_tokens : 1) - 1) - a.window;
        c.p0 += first > 0 ? first / kPage : 0;
    }
    c.p1 = min(c.p0 + pages, (len + kPage - 1) / kPage);
}

__device__ __forceinline__ Chunk chunk_of(const DecodeArgs &a, int h, int b, int part, int wave)
{
    Chunk c = chunk_start(a, h, b, part, wave);
    chunk_clamp(a, c);
    return c;
}

// True when all of the workgroup's chunks lie past the end of the context
// (wave 0's chunk, the first of them, has no page): common in ragged batches,
// where the split count follows the longest sequence.
__device__ __forceinline__ bool group_chunks_empty(const DecodeArgs &a, const Chunk &c, int wave)
{
    const int k0 = c.part * kWavesPerGroup;
    return c.p0 - (chunk_first_page(a, k0 + wave) - chunk_first_page(a, k0)) >= (c.len + kPage - 1) / kPage;
}

// The partial of such a workgroup: its rows are marked empty (m = -inf,
// l = 0), and their outputs are neither written nor read by the combine.
// Call with every thread of the workgroup.
__device__ __forceinline__ void mark_partial_empty(const DecodeArgs &a, int b, int h, int part)
{
    const int G = a.group;
    const int S = a.q_tokens > 1 ? a.q_tokens : 1;
    const int64_t row0 = (static_cast<int64_t>(b) * a.partials + part) * S * a.num_q_heads + static_cast<int64_t>(h) * G;
    for (int q = threadIdx.x; q < S * G; q += kGroupThreads) {
        const int64_t row = row0 + static_cast<int64_t>(q / G) * a.num_q_heads + q % G;
        *reinterpret_cast<float2 *>(a.ws_ml + row * 2) = make_float2(-INFINITY, 0.0f);
    }
}

// First token of the context the lane's query column sees (0 without a
// window), for a column whose prefix ends `shortfall` tokens before len.
__device__ __forceinline__ int column_first_token(const DecodeArgs &a, int len, int shortfall)
{
    const int first = len - shortfall - a.window;
    return (a.window > 0 && first > 0) ? first : 0;
}

__device__ __forceinline__ int ids_from(const DecodeArgs &a, const int32_t *ptab, int p0, int pages, int lane)
{
    const int end = min(p0 + pages, a.max_pages);
    return p0 + lane < end ? ptab[p0 + lane] : -1;
}

// The chunk's page ids, loaded from its unshifted start (a chunk_start
// value) so that the load waits for nothing but the kernel arguments.
__device__ __forceinline__ int chunk_ids(const DecodeArgs &a, const Chunk &c, int wave, int lane)
{
    const int k = c.part * kWavesPerGroup + wave;
    return ids_from(a, c.ptab, chunk_first_page(a, k), chunk_pages(a, k), lane);
}

// After chunk_clamp: only a window moves the start (by an amount that
// depends on the length), and then the ids are loaded again from the moved
// start.
__device__ __forceinline__ int chunk_ids_moved(const DecodeArgs &a, const Chunk &c, int wave, int lane, int ids)
{
    const int k = c.part * kWavesPerGroup + wave;
    if (a.window > 0 && c.p0 != chunk_first_page(a, k))
        ids = ids_from(a, c.ptab, c.p0, chunk_pages(a, k), lane);
    return ids;
}

// The step's own token (decode with append): the one wave whose chunk holds
// position len - 1 quantises the sequence's new K and V rows for its KV head
// and stores them before it copies any page.  Its copy of that page must be
// issued after the stores have completed: when the page is the chunk's first
// one, the wave waits for them here; otherwise the page loop's first wait
// (which leaves only the first page's copies outstanding, and vector memory
// operations complete in issue order) already covers them, and the stores'
// latency overlaps the first pages' copies.  Only this wave touches that
// (page, KV head) block in the kernel.
// A length past the page table (max_pages * 64) appends nothing: the
// attention clamps it, but the token's position is not in the table.
template <int D, bool FP8>
__device__ __forceinline__ void append_if_last_chunk(const DecodeArgs &a, const Chunk &c, int lane)
{
    const CacheGeom &g = a.geom;
    const int last = c.len - 1;
    if (last < 0 || last / kPage < c.p0 || last / kPage >= c.p1)
        return;
    if (a.seq_lens[c.b] > a.max_pages * kPage)
        return;
    const int id = c.ptab[last / kPage];
    if (id < 0 || id >= g.num_pages)
        return;
    uint8_t *base = a.cache_w + static_cast<int64_t>(id) * g.page_stride + c.h * g.head_stride;
    const int64_t row = (static_cast<int64_t>(c.b) * g.num_kv_heads + c.h) * D;
    quant::append_token_in_wave<D, FP8>(g, a.k_new + row, a.v_new + row, base, last % kPage, lane);
    if (last / kPage == c.p0)
        wait_vmem_at_most<0>();
}

}  // namespace mfma
}  // namespace fp4kv
