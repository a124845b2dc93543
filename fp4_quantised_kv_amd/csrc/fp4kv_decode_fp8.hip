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
// With one fp16 scale per (token, KV head) (template argument TS) a lane's
// 8 tokens of a half page -- its rows of the two score tiles, and its B
// operand of the value product -- are 8 consecutive tokens, so their K and V
// scales are 16 contiguous bytes each: the K scale multiplies the token's
// score after the product; the V scale multiplies its probability, taken
// relative to a running reference R (the largest V scale seen, moved up with
// the accumulators like the softmax max) so that p * s_v / R stays in fp16's
// range; the partials are multiplied by R at the end.  The softmax
// denominator still sums the unscaled probabilities.
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
    uint32_t s;          // per-token scales: lanes 0-7 the K plane, 8-15 the V plane, 16 bytes each
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
    o.s = static_cast<uint32_t>(lane < 8 ? g.k_scales_off : g.v_scales_off) + 16u * (lane & 7);
    return o;
}

// Per-token scales: the K slot grows by 128 bytes and holds, past the half
// page's K codes, the whole page's K scales (kScaleAt) and V scales
// (kScaleAt + 128), copied once per page with half 0.
constexpr int kScaleAt = 4096;
template <bool TS>
constexpr int k_slot_bytes() { return TS ? kSlotBytes + 128 : kSlotBytes; }

// Fp16 element k of 8 packed in a uint4, as a float.
__device__ __forceinline__ float fp16_at(const uint4 &w, int k)
{
    const uint32_t d = k < 2 ? w.x : k < 4 ? w.y : k < 6 ? w.z : w.w;
    const uint16_t h = static_cast<uint16_t>((k & 1) ? (d >> 16) : (d & 0xFFFFu));
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Running reference of the V scales (see the file comment).
struct VRef {
    float r, rcp;
};

// Weights s_v / R of the lane's 8 tokens t0 .. t0+7 (0 at or past `valid`:
// never-written slots may hold any bytes), first moving R up to the largest
// of the half page's scales if that exceeds it; every lane sees the same
// maximum (the lanes of one column cover the half page's 32 tokens).
template <int D>
__device__ __forceinline__ void v_weights(const uint4 &vs, int t0, int valid, VRef &ref, SplitState<D> &st,
                                          float (&wv)[8])
{
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        wv[k] = t0 + k < valid ? fp16_at(vs, k) : 0.0f;
        mx = fmaxf(mx, wv[k]);
    }
    mx = xor_max(mx);
    if (mx > ref.r) {
        const float a = ref.r / mx;
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
            st.acc[t] *= a;
        ref.r = mx;
        ref.rcp = 1.0f / mx;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
        wv[k] *= ref.rcp;
}

// The value product's B operand for per-token V scales: p = pf + pl (exact)
// times the weights, split again into hi + lo fp16 parts.
__device__ __forceinline__ void scale_probs(const half8_t &pf, const half8_t &pl, const float (&wv)[8],
                                            half8_t &vf, half8_t &vl)
{
    float minus_one = -1.0f;
    asm volatile("" : "+s"(minus_one));
    float p[8], q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        p[e] = (static_cast<float>(pf[e]) + static_cast<float>(pl[e])) * wv[e];
    vf = cat(pk_rtz(p[0], p[1]), pk_rtz(p[2], p[3]), pk_rtz(p[4], p[5]), pk_rtz(p[6], p[7]));
#pragma unroll
    for (int e = 0; e < 8; ++e)
        q[e] = __builtin_fmaf(static_cast<float>(vf[e]), minus_one, p[e]);
    vl = cat(pk_rtz(q[0], q[1]), pk_rtz(q[2], q[3]), pk_rtz(q[4], q[5]), pk_rtz(q[6], q[7]));
}

// Half page h of K: tiles 2h, 2h+1 (tile t starts 4t token rows past tile
// 0; part 1 is 32 token rows past part 0).  Slot layout: copy (tile i, part
// p) at (2i + p) * 1024.  With per-token scales, half 0 adds a fifth copy
// (lanes 0-15): the page's 128-byte K and V scale planes, whole (two copies
// of half planes would fetch each plane's lines twice under the
// non-temporal hint).
template <bool TS>
__device__ __forceinline__ void stage_k8(const uint8_t *blk, const Fp8Offsets &o, int h, uint8_t *slot, int lane)
{
    const uint8_t *k = blk + o.k + h * 8 * kD;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int p = 0; p < 2; ++p)
            __builtin_amdgcn_global_load_lds(k + (4 * i + 32 * p) * kD, slot + (2 * i + p) * 1024, 16, 0, kStream);
    if constexpr (TS) {
        if (h == 0 && lane < 16)
            __builtin_amdgcn_global_load_lds(blk + o.s, slot + kScaleAt, 16, 0, kStream);
    }
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
template <bool TS>
__device__ __forceinline__ void scores8(const uint8_t *slot, int col, int jj, int h, int lo, int valid,
                                        const half8_t (&qf)[kD / 32], const uint4 &ks, float (&z)[2][4])
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
        for (int e = 0; e < 4; ++e) {
            const float sc = TS ? acc[e] * fp16_at(ks, 4 * i + e) : acc[e];
            z[i][e] = (16 * jj + 8 * h + 4 * i + e < valid && 16 * jj + 8 * h + 4 * i + e >= lo) ? sc : -INFINITY;
        }
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
template <bool TS>
__device__ __forceinline__ void fp8_pages(uint8_t *__restrict__ kslot, uint8_t *__restrict__ vslot,
                                          const DecodeArgs &a, const Fp8Offsets &o, int lane, int col, int jj, int h,
                                          int p0, int p1, int len, int shortfall, int first, const int32_t *ptab,
                                          int ids, int pid,
                                          const half8_t (&qf)[kD / 32], float zscale, SplitState<kD> &st,
                                          VRef &ref)
{
    constexpr int kKCopies0 = TS ? kCopies + 1 : kCopies;  // copies of half 0 of K (with the scales)
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

            // K: outstanding now are this half's K (and scale) copies, then V's
            if (cur)
                wait_vmem_at_most<kCopies>();
            uint4 ks = {0u, 0u, 0u, 0u}, vs = {0u, 0u, 0u, 0u};
            if constexpr (TS) {
                // the lane's tokens 16jj + 8hf .. +7
                ks = *reinterpret_cast<const uint4 *>(kslot + kScaleAt + 32 * jj + 16 * hf);
                vs = *reinterpret_cast<const uint4 *>(kslot + kScaleAt + 128 + 32 * jj + 16 * hf);
            }
            float z[2][4];
            scores8<TS>(kslot, col, jj, hf, first - pg * kPage, min(kPage, len - pg * kPage - shortfall), qf, ks, z);
            __builtin_amdgcn_s_waitcnt(kWaitLds);
            if (next)
                stage_k8<TS>(nblk, o, nh, kslot, lane);
            if (cur) {
                softmax_tiles<kD, 2>(z, st, zscale, pf, pl);
                if constexpr (TS) {
                    float wv[8];
                    v_weights<kD>(vs, 16 * jj + 8 * hf, valid, ref, st, wv);
                    scale_probs(pf[0], pl[0], wv, pf[0], pl[0]);
                }
            }

            // V: outstanding now are this half's V then the next half's K
            if (next) {
                if (hf == 1)
                    wait_vmem_at_most<kKCopies0>();        // the next half is half 0 of the next page
                else
                    wait_vmem_at_most<kCopies>();
            } else {
                wait_vmem_at_most<0>();
            }
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

template <bool APPEND, bool TS>
__global__ __launch_bounds__(kGroupThreads) void decode_split_fp8(DecodeArgs a)
{
    static_assert(kScaleAt + 256 <= k_slot_bytes<true>(), "a page's scales fit the K slot");
    static_assert(kWavesPerGroup * (k_slot_bytes<TS>() + kSlotBytes) <= 40 * 1024, "four workgroups per CU");
    static_assert(merge_area_bytes<kD>() <= 2 * kSlotBytes, "merge area layout");
    static_assert(8 * kD * 4 + 128 <= kSlotBytes, "merge area must fit the slots");
    static_assert(kWavesPerGroup * 2 * kSlotBytes <= 40 * 1024, "four workgroups per CU");

    __shared__ __attribute__((aligned(16))) uint8_t kslots[kWavesPerGroup][k_slot_bytes<TS>()];
    __shared__ __attribute__((aligned(16))) uint8_t vslots[kWavesPerGroup][kSlotBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;
    const int jj = lane >> 4;
    const CacheGeom &g = a.geom;

    // grid (KV head, sequence, partial), as for the FP4 kernel
    Chunk c = chunk_start(a, blockIdx.x, blockIdx.y, blockIdx.z, wave);
    int ids = chunk_ids(a, c, wave, lane);
    uint32_t qbits[kD / 8];
    load_q_bits<kD>(a, c.b, c.h, col, jj, qbits);
    // the length only now, so that its load overlaps the ones above
    __builtin_amdgcn_sched_barrier(0);
    chunk_clamp(a, c);
    ids = chunk_ids_moved(a, c, wave, lane, ids);
    if (!a.out && group_chunks_empty(a, c, wave)) {     // every chunk of the workgroup past the context
        mark_partial_empty(a, c.b, c.h, c.part);
        return;
    }
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
        stage_k8<TS>(blk, o, 0, kslots[wave], lane);
        stage_v8(blk, o, 0, vslots[wave]);
    }
    const int shortfall = column_shortfall(a, col);
    VRef ref = {0.0f, 0.0f};
    fp8_pages<TS>(kslots[wave], vslots[wave], a, o, lane, col, jj, c.h, c.p0, c.p1, c.len, shortfall,
                  column_first_token(a, c.len, shortfall), c.ptab, ids, pid, qf, zscale, st, ref);

    // the V tensor's scale (or the reference the per-token ones were taken
    // against) multiplies every value, so it multiplies o
    const float vsc = TS ? ref.r : g.v_scale;
#pragma unroll
    for (int t = 0; t < kD / 16; ++t)
        st.acc[t] *= vsc;
    auto area = [&](int w) { return MergeArea<kD>(kslots[w], vslots[w]); };
    state_to_area<kD>(area(wave), st, col, jj, query_columns(a));
    merge_waves_and_store<kD>(area, a, c.b, c.h, c.part);
}

// Head dim 64: operands loaded straight into registers (no LDS staging).
// Score tile t of half page h (t = 2h + i): the lane's token row is
// tile_token(t, col), and its 16 channels 16jj .. 16jj+15 -- the A operands
// of the two MFMAs, in the query operand's channel order -- are one 16-byte
// load.  Values: the lane's two channels 32u + 2col, +1 of the half page's
// tokens 16jj + 8h .. +7 are one 16-byte row pair, as in the staged kernel;
// with per-token scales, so are the 8 K and the 8 V scales of those tokens.
template <bool APPEND, bool TS>
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
    if (!a.out && group_chunks_empty(a, c, wave)) {     // every chunk of the workgroup past the context
        mark_partial_empty(a, c.b, c.h, c.part);
        return;
    }
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
    VRef ref = {0.0f, 0.0f};
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
            uint4 ks = {0u, 0u, 0u, 0u}, vs = {0u, 0u, 0u, 0u};
            if constexpr (TS) {
                ks = *reinterpret_cast<const uint4 *>(blk + g.k_scales_off + 32 * jj + 16 * hf);
                vs = *reinterpret_cast<const uint4 *>(blk + g.v_scales_off + 32 * jj + 16 * hf);
            }
            float z[2][4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8(kx[i].x, kx[i].y), qf[0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp8x8(kx[i].z, kx[i].w), qf[1], acc, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tok = 16 * jj + 8 * hf + 4 * i + e;
                    const float sc = TS ? acc[e] * fp16_at(ks, 4 * i + e) : acc[e];
                    z[i][e] = (tok < hi && tok >= lo) ? sc : -INFINITY;
                }
            }
            half8_t pf[1], pl[1];
            softmax_tiles<D, 2>(z, st, zscale, pf, pl);
            if constexpr (TS) {
                float wv[8];
                v_weights<D>(vs, 16 * jj + 8 * hf, valid, ref, st, wv);
                scale_probs(pf[0], pl[0], wv, pf[0], pl[0]);
            }
#pragma unroll
            for (int u = 0; u < D / 32; ++u)
                values8<D>(vx[u], u, jj, hf, valid, pf[0], pl[0], st);
        }
    }
    const float vsc = TS ? ref.r : g.v_scale;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
        st.acc[t] *= vsc;
    auto area = [&](int w) { return MergeArea<D>(areas[w]); };
    state_to_area<D>(area(wave), st, col, jj, query_columns(a));
    merge_waves_and_store<D>(area, a, c.b, c.h, c.part);
}

}  // namespace

namespace {

template <bool APPEND, bool TS>
void launch_fp8(const DecodeArgs &a, hipStream_t stream)
{
    const dim3 grid(a.geom.num_kv_heads, a.batch, a.partials);
    if (a.geom.head_dim == 64)
        decode_split_fp8_d64<APPEND, TS><<<grid, kGroupThreads, 0, stream>>>(a);
    else
        decode_split_fp8<APPEND, TS><<<grid, kGroupThreads, 0, stream>>>(a);
}

}  // namespace

hipError_t launch_split_fp8(const DecodeArgs &a, hipStream_t stream)
{
    const bool append = a.k_new != nullptr;
    if (a.geom.token_scales)
        append ? launch_fp8<true, true>(a, stream) : launch_fp8<false, true>(a, stream);
    else
        append ? launch_fp8<true, false>(a, stream) : launch_fp8<false, false>(a, stream);
    return hipGetLastError();
}

}  // namespace fp4kv
