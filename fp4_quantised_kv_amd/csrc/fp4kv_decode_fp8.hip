// Split-K decode attention over an FP8 E4M3 cache with one scale per tensor
// ("Quantising the KV cache", Concept section, results table: FP8 E4M3, one
// scale per tensor, 8 bits per number), on the CDNA4 matrix cores.
//
// The structure is the FP4 kernel's (fp4kv_decode_mfma.hip): workgroups of
// four waves, one context chunk per wave, scores S^T = K^ Q^T and values
// O^T = V^T P^T on v_mfma_f32_16x16x32_f16, P as hi + lo fp16 parts, an
// online softmax with a lazily moved reference max, an LDS merge into one
// partial per workgroup.  What differs:
//   - an E4M3 code converts to fp16 exactly with no scale multiply (every
//     E4M3 value is an fp16 value); the K tensor's scale is folded into the
//     softmax scale on the host, the V tensor's scale into the partials;
//   - pages are staged in 32-token halves (score tiles 2h and 2h+1, and the
//     tokens 16j + 8h .. 16j + 8h + 7 of the value product's k-block h), so
//     that a half page of K (4 KB) and of V (4 KB) fill the same LDS slots a
//     whole FP4 page does and four workgroups still fit a CU;
//   - V is stored in [slice][half][channel][8 tokens] rows, so a lane's two
//     channels of a half page are 16 contiguous bytes.
#include <cstdint>

#include <hip/hip_runtime.h>

#include "fp4kv_internal.h"
#include "fp4kv_merge.h"
#include "fp4kv_mfma_util.h"

namespace fp4kv {
namespace {

using namespace mfma;

constexpr int kD = 128;
constexpr int kSlotBytes = 4096 + 128;    // half a page of K or V; the merge area needs 8*D*4 + 128
constexpr int kCopies = 4;                // direct-to-LDS instructions per half-page copy of K or of V

// Per-lane byte offsets inside a block for half page 0; half h adds 8h
// token rows (K) or one 8-token row block (V).
struct Fp8Offsets {
    uint32_t k, v;
};

// K copies fetch whole 128-byte token rows: in copy (tile i, part p), lane l
// fetches 16-byte chunk l % 8 of the row of tile row 8p + l / 8, i.e. token
// 32p + 16(l / 32) + 4t + (l / 8) % 4 (t = the tile) -- with the non-temporal
// hint a row split over two copies could be fetched twice.  The lane that
// needs chunks 2jj, 2jj+1 of tile row col finds them at lane slots
// 8(col % 8) + 2jj, +1 of copy (i, col / 8).
__device__ __forceinline__ Fp8Offsets fp8_offsets(const CacheGeom &g, int lane, int col, int jj)
{
    Fp8Offsets o;
    o.k = static_cast<uint32_t>(g.k_codes_off) +
          (16u * (lane >> 5) + ((lane >> 3) & 3)) * kD + (lane & 7) * 16u;
    // V: channels 2col, 2col+1 of slice jj, 8 tokens each
    o.v = static_cast<uint32_t>(g.v_codes_off) + ((jj * 2u) * kD + 2u * col) * 8u;
    return o;
}

// Half page h of K: tiles 2h, 2h+1 (tile t starts 4t token rows past tile
// 0; part 1 is 32 token rows past part 0).  Slot layout: copy (tile i, part
// p) at (2i + p) * 1024.
__device__ __forceinline__ void stage_k8(const uint8_t *blk, const Fp8Offsets &o, int h, uint8_t *slot)
{
    const uint8_t *k = blk + o.k + h * 8 * kD;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int p = 0; p < 2; ++p)
            __builtin_amdgcn_global_load_lds(k + (4 * i + 32 * p) * kD, slot + (2 * i + p) * 1024, 16, 0, kStream);
}

// Half page h of V: pair block u (32 channels, 256 bytes of rows) at u*1024.
__device__ __forceinline__ void stage_v8(const uint8_t *blk, const Fp8Offsets &o, int h, uint8_t *slot)
{
    const uint8_t *v = blk + o.v + h * kD * 8;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        __builtin_amdgcn_global_load_lds(v + 256 * u, slot + u * 1024, 16, 0, kStream);
}

// 8 E4M3 codes (two dwords, in order) -> fp16.
__device__ __forceinline__ half8_t fp8x8(uint32_t a, uint32_t b)
{
    return cat(fp8x2<false>(a), fp8x2<true>(a), fp8x2<false>(b), fp8x2<true>(b));
}

// Scores of half page h: tiles 2h + i, A operand of MFMA m = channels
// 32jj + 8m .. +7 of the lane's token, the same channel order as the query
// operand.  Tokens outside lo .. valid-1 (the lane's query column's window
// in this page) get -inf.
__device__ __forceinline__ void scores8(const uint8_t *slot, int col, int jj, int h, int lo, int valid,
                                        const half8_t (&qf)[kD / 32], float (&z)[2][4])
{
    const int at = (col >> 3) * 1024 + (((col & 7) << 3) + 2 * jj) * 16;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint4 a = *reinterpret_cast<const uint4 *>(slot + 2 * i * 1024 + at);
        const uint4 b = *reinterpret_cast<const uint4 *>(slot + 2 * i * 1024 + at + 16);
        float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8(a.x, a.y), qf[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8(a.z, a.w), qf[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8(b.x, b.y), qf[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8(b.z, b.w), qf[3], acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            z[i][e] = (16 * jj + 8 * h + 4 * i + e < valid && 16 * jj + 8 * h + 4 * i + e >= lo) ? acc[e] : -INFINITY;
    }
}

// Values of half page h, pair block u: the lane's 16 bytes are channel c's
// 8 tokens then channel c+1's (c = 32u + 2col); codes of tokens at or past
// `valid` are zeroed so that never-written slots (possibly NaN codes) add
// exact zeros.
template <int D = kD>
__device__ __forceinline__ void values8(uint4 w, int u, int jj, int h, int valid, const half8_t &pf,
                                        const half8_t &pl, SplitState<D> &st)
{
    if (valid < kPage) {
        const int t0 = 16 * jj + 8 * h;
        w.x = keep_valid_bytes(w.x, t0, valid);
        w.y = keep_valid_bytes(w.y, t0 + 4, valid);
        w.z = keep_valid_bytes(w.z, t0, valid);
        w.w = keep_valid_bytes(w.w, t0 + 4, valid);
    }
    const half8_t ev = fp8x8(w.x, w.y), od = fp8x8(w.z, w.w);
    float4_t &ae = st.acc[2 * u];
    float4_t &ao = st.acc[2 * u + 1];
    ae = __builtin_amdgcn_mfma_f32_16x16x32_f16(ev, pf, ae, 0, 0, 0);
    ae = __builtin_amdgcn_mfma_f32_16x16x32_f16(ev, pl, ae, 0, 0, 0);
    ao = __builtin_amdgcn_mfma_f32_16x16x32_f16(od, pf, ao, 0, 0, 0);
    ao = __builtin_amdgcn_mfma_f32_16x16x32_f16(od, pl, ao, 0, 0, 0);
}

// The page loop over half pages.  On entry `ids` holds the page ids of
// pages p0 .. p0+63 (one per lane) and the copies of half 0 of page p0 (id
// `pid`) have been issued, K then V, if it is live.  Slots are
// restrict-qualified so that the compiler's LDS-copy wait tracking knows
// they never alias.
__device__ __forceinline__ void fp8_pages(uint8_t *__restrict__ kslot, uint8_t *__restrict__ vslot,
                                          const DecodeArgs &a, const Fp8Offsets &o, int lane, int col, int jj, int h,
                                          int p0, int p1, int len, int shortfall, int first, const int32_t *ptab,
                                          int ids, int pid,
                                          const half8_t (&qf)[kD / 32], float zscale, SplitState<kD> &st)
{
    const CacheGeom &g = a.geom;
    auto live_page = [&](int id) { return id >= 0 && id < g.num_pages; };
    auto block_of = [&](int id) {
        return a.cache + static_cast<int64_t>(id) * g.page_stride + h * g.head_stride;
    };
    int base = p0;
    for (int pg = p0; pg < p1; ++pg) {
        const int nxt = pg + 1;
        if (nxt < p1 && nxt - base == 64) {
            base = nxt;
            ids = (base + lane < p1) ? ptab[base + lane] : -1;
            wait_vmem_at_most<0>();
        }
        const int pid_next = nxt < p1 ? __builtin_amdgcn_readlane(ids, nxt - base) : -1;
        const bool cur = live_page(pid);
        const int valid = min(kPage, len - pg * kPage);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            // the half page after this one: the other half of this page, or
            // half 0 of the next page
            const bool next = hf == 0 ? cur : live_page(pid_next);
            const uint8_t *nblk = hf == 0 ? block_of(pid) : block_of(pid_next);
            const int nh = hf == 0 ? 1 : 0;
            half8_t pf[1], pl[1];

            // K: outstanding now are this half's K then V copies
            if (cur)
                wait_vmem_at_most<kCopies>();
            float z[2][4];
            scores8(kslot, col, jj, hf, first - pg * kPage, min(kPage, len - pg * kPage - shortfall), qf, z);
            __builtin_amdgcn_s_waitcnt(kWaitLds);
            if (next)
                stage_k8(nblk, o, nh, kslot);
            if (cur)
                softmax_tiles<kD, 2>(z, st, zscale, pf, pl);

            // V: outstanding now are this half's V then the next half's K
            if (next)
                wait_vmem_at_most<kCopies>();
            else
                wait_vmem_at_most<0>();
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint4 w = *reinterpret_cast<const uint4 *>(vslot + u * 1024 + lane * 16);
                __builtin_amdgcn_s_waitcnt(kWaitLds);
                if (u == 3 && next)
                    stage_v8(nblk, o, nh, vslot);
                if (cur)
                    values8(w, u, jj, hf, valid, pf[0], pl[0], st);
            }
        }
        pid = pid_next;
    }
}

template <bool APPEND>
__global__ __launch_bounds__(kGroupThreads) void decode_split_fp8(DecodeArgs a)
{
    static_assert(merge_area_bytes<kD>() <= 2 * kSlotBytes, "merge area layout");
    static_assert(8 * kD * 4 + 128 <= kSlotBytes, "merge area must fit the slots");
    static_assert(kWavesPerGroup * 2 * kSlotBytes <= 40 * 1024, "four workgroups per CU");

    __shared__ __attribute__((aligned(16))) uint8_t kslots[kWavesPerGroup][kSlotBytes];
    __shared__ __attribute__((aligned(16))) uint8_t vslots[kWavesPerGroup][kSlotBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;
    const int jj = lane >> 4;
    const CacheGeom &g = a.geom;

    // grid (KV head, sequence, partial), as for the FP4 kernel
    const Chunk c = chunk_of(a, blockIdx.x, blockIdx.y, blockIdx.z, wave);
    const int ids = chunk_ids(a, c, lane);
    uint32_t qbits[kD / 8];
    load_q_bits<kD>(a, c.b, c.h, col, jj, qbits);
    half8_t qf[kD / 32];
    float zscale;
    make_q_operand<kD>(qbits, a.scale_log2e, qf, zscale);   // scale_log2e includes the K tensor's scale

    if constexpr (APPEND)
        append_if_last_chunk<kD, true>(a, c, lane);

    SplitState<kD> st;
    init_state(st);
    const Fp8Offsets o = fp8_offsets(g, lane, col, jj);
    const int pid = c.p0 < c.p1 ? __builtin_amdgcn_readlane(ids, 0) : -1;
    if (pid >= 0 && pid < g.num_pages) {
        const uint8_t *blk = a.cache + static_cast<int64_t>(pid) * g.page_stride + c.h * g.head_stride;
        stage_k8(blk, o, 0, kslots[wave]);
        stage_v8(blk, o, 0, vslots[wave]);
    }
    const int shortfall = column_shortfall(a, col);
    fp8_pages(kslots[wave], vslots[wave], a, o, lane, col, jj, c.h, c.p0, c.p1, c.len, shortfall,
              column_first_token(a, c.len, shortfall), c.ptab, ids, pid, qf, zscale, st);

    // the V tensor's scale multiplies every value, so it multiplies o
#pragma unroll
    for (int t = 0; t < kD / 16; ++t)
        st.acc[t] *= g.v_scale;
    auto area = [&](int w) { return MergeArea<kD>(kslots[w], vslots[w]); };
    state_to_area<kD>(area(wave), st, col, jj, query_columns(a));
    merge_waves_and_store<kD>(area, a, c.b, c.h, c.part);
}

// Head dim 64: operands loaded straight into registers (no LDS staging).
// Score tile t of half page h (t = 2h + i): the lane's token row is
// tile_token(t, col), and its 16 channels 16jj .. 16jj+15 -- the A operands
// of the two MFMAs, in the query operand's channel order -- are one 16-byte
// load.  Values: the lane's two channels 32u + 2col, +1 of the half page's
// tokens 16jj + 8h .. +7 are one 16-byte row pair, as in the staged kernel.
template <bool APPEND>
__global__ __launch_bounds__(kGroupThreads) void decode_split_fp8_d64(DecodeArgs a)
{
    constexpr int D = 64;
    __shared__ __attribute__((aligned(16))) uint8_t areas[kWavesPerGroup][merge_area_bytes<D>()];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;
    const int jj = lane >> 4;
    const CacheGeom &g = a.geom;

    const Chunk c = chunk_of(a, blockIdx.x, blockIdx.y, blockIdx.z, wave);
    uint32_t qbits[D / 8];
    load_q_bits<D>(a, c.b, c.h, col, jj, qbits);
    half8_t qf[D / 32];
    float zscale;
    make_q_operand<D>(qbits, a.scale_log2e, qf, zscale);
    if constexpr (APPEND) {
        append_if_last_chunk<D, true>(a, c, lane);
        wait_vmem_at_most<0>();                         // the page loads below are issued without a wait
    }
    const int shortfall = column_shortfall(a, col);
    const int first = column_first_token(a, c.len, shortfall);

    SplitState<D> st;
    init_state(st);
    for (int pg = c.p0; pg < c.p1; ++pg) {
        const int id = c.ptab[pg];
        if (id < 0 || id >= g.num_pages)                // skipped, like the other kernels
            continue;
        const uint8_t *blk = a.cache + static_cast<int64_t>(id) * g.page_stride + c.h * g.head_stride;
        const int valid = min(kPage, c.len - pg * kPage);
        const int lo = first - pg * kPage, hi = min(kPage, c.len - pg * kPage - shortfall);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            uint4 kx[2], vx[D / 32];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                kx[i] = *reinterpret_cast<const uint4 *>(blk + g.k_codes_off + tile_token(2 * hf + i, col) * D +
                                                          16 * jj);
#pragma unroll
            for (int u = 0; u < D / 32; ++u)
                vx[u] = *reinterpret_cast<const uint4 *>(blk + g.v_codes_off +
                                                          ((jj * 2 + hf) * D + 32 * u + 2 * col) * 8);
            float z[2][4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8(kx[i].x, kx[i].y), qf[0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8(kx[i].z, kx[i].w), qf[1], acc, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tok = 16 * jj + 8 * hf + 4 * i + e;
                    z[i][e] = (tok < hi && tok >= lo) ? acc[e] : -INFINITY;
                }
            }
            half8_t pf[1], pl[1];
            softmax_tiles<D, 2>(z, st, zscale, pf, pl);
#pragma unroll
            for (int u = 0; u < D / 32; ++u)
                values8<D>(vx[u], u, jj, hf, valid, pf[0], pl[0], st);
        }
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
        st.acc[t] *= g.v_scale;
    auto area = [&](int w) { return MergeArea<D>(areas[w]); };
    state_to_area<D>(area(wave), st, col, jj, query_columns(a));
    merge_waves_and_store<D>(area, a, c.b, c.h, c.part);
}

}  // namespace

hipError_t launch_split_fp8(const DecodeArgs &a, hipStream_t stream)
{
    if (a.geom.head_dim == 64) {
        const dim3 grid(a.geom.num_kv_heads, a.batch, a.partials);
        if (a.k_new)
            decode_split_fp8_d64<true><<<grid, kGroupThreads, 0, stream>>>(a);
        else
            decode_split_fp8_d64<false><<<grid, kGroupThreads, 0, stream>>>(a);
        return hipGetLastError();
    }
    const dim3 grid(a.geom.num_kv_heads, a.batch, a.partials);
    if (a.k_new)
        decode_split_fp8<true><<<grid, kGroupThreads, 0, stream>>>(a);
    else
        decode_split_fp8<false><<<grid, kGroupThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace fp4kv
